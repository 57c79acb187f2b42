// gfx950 kernels of the verify-and-resample step of speculative sampling.
//
// A call runs three kernels on the caller's stream; the kernel boundaries
// order them, so no work-group ever waits for another:
//
//   chunk_kernel    grid (sequence, logit row, chunk).  Every used logit row
//                   (target positions 0..K_b, draft positions 0..K_b-1) is
//                   split into S chunks of at most 32768 bf16 / 16384 fp32
//                   logits; each work-group streams its chunk from HBM into
//                   registers exactly once and reduces it: maximum, sum of
//                   2^((x - m) c2), the candidate list of the nucleus / top-k
//                   threshold search, the greedy argmax.  One instance per
//                   sampling mode keeps the registers of each mode's loop
//                   minimal.
//   merge_kernel    grid (sequence, logit row).  Log-sum-exp merge of the
//                   chunks, radix selection of the threshold over the
//                   candidates (cached in LDS), kept mass, the probability of
//                   the row's draft token, and for target rows the kept set
//                   in vocabulary order with its probabilities.
//   final_kernel    grid (sequence).  Accept walk, first rejection, resample
//                   from normalize((q - p)+) or the bonus draw, outputs.
//
// The step follows the pages' rule (FDE Interviews breakdown of Chen et al.,
// section 01 and its figure; paperlayer.ai summary of arXiv 2302.01318,
// "Modified Rejection Sampling"): keep d_t with probability
// min(1, q_t(d_t) / p_t(d_t)), resample the first rejection from the
// normalised positive part of q - p, else draw a bonus token from the
// target's last position; sampling controls are applied to both models
// before the rejection step.  The pages describe no GPU kernel; everything
// below is this library's own design for gfx950.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sv_internal.h"

namespace sv {
namespace {

constexpr float kInf = __builtin_inff();
constexpr int kWave = 64;
constexpr float kMaxFinite = 3.402823466e38f;
constexpr double kLog2e = 1.4426950408889634074;
// Fixed-point scale of masses (units of the row's largest term): integer
// accumulation makes histogram sums independent of atomic order.
constexpr double kFix = 1099511627776.0;  // 2^40
constexpr double kWindow = 1e-6;
// Nucleus candidates: tokens whose term is within 2^-10 of the chunk's
// largest term (on the pages' workloads a window of 2^-8 to 2^-9.4 already
// covers the nucleus; a list that overflows is retried with 2^-8, 2^-6).
constexpr float kCandLog2 = 10.0f;

constexpr uint32_t kPurposeAccept = 0, kPurposeResample = 1, kPurposeBonus = 2;
constexpr uint32_t kErrBits = SV_ST_TOKEN | SV_ST_NONFINITE | SV_ST_EMPTY | SV_ST_PARAM;

// ------------------------------------------------------------ Philox -----
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of two
// 32x32->64 multiplies whose halves are mixed with the other counter words
// and a Weyl-sequence key.  Only word 0 of the output is used.
__device__ __forceinline__ uint32_t philox_word0(uint64_t seed, uint64_t g, uint32_t t,
                                                 uint32_t purpose) {
  uint32_t c0 = (uint32_t)g, c1 = t, c2 = purpose, c3 = (uint32_t)(g >> 32);
  uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t hi_a = __umulhi(0xD2511F53u, c0), lo_a = 0xD2511F53u * c0;
    const uint32_t hi_b = __umulhi(0xCD9E8D57u, c2), lo_b = 0xCD9E8D57u * c2;
    const uint32_t n0 = hi_b ^ c1 ^ k0;
    const uint32_t n2 = hi_a ^ c3 ^ k1;
    c0 = n0;
    c1 = lo_b;
    c2 = n2;
    c3 = lo_a;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c0;
}

__device__ __forceinline__ double uniform24(uint64_t seed, uint64_t g, uint32_t t, uint32_t purpose) {
  return (double)(philox_word0(seed, g, t, purpose) >> 8) * (1.0 / 16777216.0);
}

// ------------------------------------------------------- logit access ----
template <int DT>
struct Fmt {
  static constexpr int VE = DT == SV_BF16 ? 8 : 4;  // logits per 16-byte vector
  static constexpr int ES = DT == SV_BF16 ? 2 : 4;  // bytes per logit
};

template <int DT>
__device__ __forceinline__ float elem(const uint4& v, int k) {
  if constexpr (DT == SV_BF16) {
    const uint32_t w = k < 2 ? v.x : (k < 4 ? v.y : (k < 6 ? v.z : v.w));
    return (k & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
  } else {
    const uint32_t w = k == 0 ? v.x : (k == 1 ? v.y : (k == 2 ? v.z : v.w));
    return __uint_as_float(w);
  }
}

template <int DT>
__device__ __forceinline__ float load_logit(const void* row, int e) {
  if constexpr (DT == SV_BF16)
    return __uint_as_float((uint32_t)static_cast<const uint16_t*>(row)[e] << 16);
  else
    return static_cast<const float*>(row)[e];
}

// The vector of VE logits starting at e0 (< c1), with -inf past c1.
template <int DT, bool VEC>
__device__ __forceinline__ uint4 load_vec(const char* row, int e0, int c1) {
  constexpr int VE = Fmt<DT>::VE, ES = Fmt<DT>::ES;
  if constexpr (VEC) {
    return *reinterpret_cast<const uint4*>(row + (size_t)e0 * ES);
  } else {
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (DT == SV_BF16) {
        const int e = e0 + 2 * j;
        const uint16_t* r16 = reinterpret_cast<const uint16_t*>(row);
        const uint32_t lo = e < c1 ? (uint32_t)r16[e] : 0xff80u;
        const uint32_t hi = e + 1 < c1 ? (uint32_t)r16[e + 1] : 0xff80u;
        w[j] = lo | (hi << 16);
      } else {
        const int e = e0 + j;
        w[j] = e < c1 ? reinterpret_cast<const uint32_t*>(row)[e] : 0xff800000u;
      }
    }
    (void)VE;
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Order-preserving key of a float (-0 is folded onto +0 so equal values
// share a key).
__device__ __forceinline__ uint32_t fkey(float x) {
  const uint32_t b = __float_as_uint(x + 0.0f);
  return b ^ ((b >> 31) ? 0xFFFFFFFFu : 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k >> 31) ? (k ^ 0x80000000u) : ~k);
}

// --------------------------------------------------------- reductions ----
// Fixed-order butterflies: every lane ends with bit-identical results.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ int wave_min_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ int wave_max_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
}

struct Red {
  float f[8];
  double d[4];
  int i[4];
  unsigned long long u[4];
};

__device__ __forceinline__ float block_max(float v, Red& r) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) r.f[w] = v;
  __syncthreads();
  return fmaxf(fmaxf(r.f[0], r.f[1]), fmaxf(r.f[2], r.f[3]));
}
__device__ __forceinline__ double block_sum(double v, Red& r) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) r.d[w] = v;
  __syncthreads();
  return (r.d[0] + r.d[1]) + (r.d[2] + r.d[3]);
}
__device__ __forceinline__ int block_sum_i(int v, Red& r) {
  v = wave_sum_i(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) r.i[w] = v;
  __syncthreads();
  return (r.i[0] + r.i[1]) + (r.i[2] + r.i[3]);
}
__device__ __forceinline__ int block_min_i(int v, Red& r) {
  v = wave_min_i(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) r.i[w] = v;
  __syncthreads();
  return min(min(r.i[0], r.i[1]), min(r.i[2], r.i[3]));
}
__device__ __forceinline__ int block_max_i(int v, Red& r) {
  v = wave_max_i(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) r.i[w] = v;
  __syncthreads();
  return max(max(r.i[0], r.i[1]), max(r.i[2], r.i[3]));
}
__device__ __forceinline__ unsigned long long block_sum_u64(unsigned long long v, Red& r) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) r.u[w] = v;
  __syncthreads();
  return (r.u[0] + r.u[1]) + (r.u[2] + r.u[3]);
}

// Exclusive prefix sum over the work-group in thread order (fp64).
__device__ __forceinline__ double block_exclusive_scan(double v, double* total, Red& r) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  double inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double y = __shfl_up(inc, o);
    if (lane >= o) inc += y;
  }
  __syncthreads();
  if (lane == 63) r.d[w] = inc;
  __syncthreads();
  double base = 0.0;
  for (int j = 0; j < w; ++j) base += r.d[j];
  *total = ((r.d[0] + r.d[1]) + r.d[2]) + r.d[3];
  return base + inc - v;
}

// ---------------------------------------------------- per-sequence params --
struct SeqParams {
  int Kb, mode, topk;
  float tau, topp;
  double c2;  // log2(e) / tau
  bool valid;
};

__device__ __forceinline__ int raw_mode(const KParams& P, int b) {
  return P.mode ? (int)P.mode[b] : P.dmode;
}

__device__ __forceinline__ SeqParams load_params(const KParams& P, int b) {
  SeqParams s;
  s.Kb = P.kpr ? P.kpr[b] : P.K_max;
  s.mode = raw_mode(P, b);
  s.tau = P.temp ? P.temp[b] : P.dtemp;
  s.topk = P.topk ? P.topk[b] : P.dtopk;
  s.topp = P.topp ? P.topp[b] : P.dtopp;
  bool ok = s.Kb >= 0 && s.Kb <= P.K_max && s.mode >= 0 && s.mode <= 3;
  if (ok && s.mode != SV_GREEDY) ok = isfinite(s.tau) && s.tau > 0.0f;
  if (ok && s.mode == SV_TOPK) ok = s.topk >= 1 && s.topk <= P.V;
  if (ok && s.mode == SV_TOPP) ok = s.topp > 0.0f && s.topp <= 1.0f;
  s.valid = ok;
  // top_p = 1 keeps every token of non-zero probability; k = V keeps every
  // token: both are plain sampling.
  if (ok && s.mode == SV_TOPP && s.topp >= 1.0f) s.mode = SV_PLAIN;
  if (ok && s.mode == SV_TOPK && s.topk >= P.V) s.mode = SV_PLAIN;
  s.c2 = (ok && s.mode != SV_GREEDY) ? kLog2e / (double)s.tau : 0.0;
  return s;
}

template <int DT>
__device__ __forceinline__ const void* row_ptr(const KParams& P, int b, bool tgt, int t) {
  constexpr int ES = Fmt<DT>::ES;
  const size_t r = tgt ? ((size_t)b * (P.K_max + 1) + t) : ((size_t)b * P.K_max + t);
  return static_cast<const char*>(tgt ? P.target : P.draft) + r * (size_t)P.V * ES;
}

// Row r of a sequence: target positions 0..K_max, then draft positions.
__device__ __forceinline__ bool decode_row(const KParams& P, const SeqParams& sp, int r, bool* tgt, int* t) {
  *tgt = r <= P.K_max;
  *t = *tgt ? r : r - P.K_max - 1;
  return *tgt ? (*t <= sp.Kb) : (*t < sp.Kb);
}

// ======================================================= chunk kernel ====
//
// Each wave owns one chunk of a logit row (64 lanes x kLoads vectors) and
// reduces it on its own, with wave ballots and shuffles only: no barrier and
// no LDS, so the waves of a work-group never wait for one another.

// Loads this lane's part of chunk [c0, c1) into registers: vector i holds
// logits c0 + (i * 64 + lane) * VE + [0, VE).  Every load is issued
// unconditionally from a clamped in-bounds address and the out-of-range
// vectors are replaced by -inf afterwards, so all kLoads requests are in
// flight together.
template <int DT, bool VEC>
__device__ __forceinline__ void load_chunk(uint4 (&buf)[kLoads], const char* row, int c0, int c1, int lane) {
  constexpr int VE = Fmt<DT>::VE, ES = Fmt<DT>::ES;
  const uint32_t ninf = DT == SV_BF16 ? 0xff80ff80u : 0xff800000u;
  if constexpr (VEC) {
    // c0 and c1 are multiples of VE and c1 - c0 >= VE
    const uint4* base = reinterpret_cast<const uint4*>(row + (size_t)c0 * ES);
    if (c1 - c0 == kWave * kLoads * VE) {
      // a whole chunk: one base address and constant offsets
#pragma unroll
      for (int i = 0; i < kLoads; ++i) buf[i] = base[i * kWave + lane];
    } else {
      // the row's last chunk: clamped addresses, -inf past c1
      const int nvec = (c1 - c0) / VE;
#pragma unroll
      for (int i = 0; i < kLoads; ++i) buf[i] = base[min(i * kWave + lane, nvec - 1)];
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        const bool ok = i * kWave + lane < nvec;
        buf[i].x = ok ? buf[i].x : ninf;
        buf[i].y = ok ? buf[i].y : ninf;
        buf[i].z = ok ? buf[i].z : ninf;
        buf[i].w = ok ? buf[i].w : ninf;
      }
    }
  } else {
    const int last = c1 - 1;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int e0 = c0 + (i * kWave + lane) * VE;
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (DT == SV_BF16) {
          const int e = e0 + 2 * j;
          const uint16_t* r16 = reinterpret_cast<const uint16_t*>(row);
          uint32_t lo = r16[min(e, last)], hi = r16[min(e + 1, last)];
          lo = e < c1 ? lo : 0xff80u;
          hi = e + 1 < c1 ? hi : 0xff80u;
          w[j] = lo | (hi << 16);
        } else {
          const int e = e0 + j;
          const uint32_t v = reinterpret_cast<const uint32_t*>(row)[min(e, last)];
          w[j] = e < c1 ? v : 0xff800000u;
        }
      }
      buf[i] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

// Hides the packed logits from the optimiser between passes so that each pass
// unpacks them again instead of keeping 128 unpacked values live.
__device__ __forceinline__ void fence_regs(uint4 (&buf)[kLoads]) {
#pragma unroll
  for (int i = 0; i < kLoads; ++i)
    asm volatile("" : "+v"(buf[i].x), "+v"(buf[i].y), "+v"(buf[i].z), "+v"(buf[i].w));
}

// Number of the chunk's elements >= cut (wave ballots).
template <int DT>
__device__ __forceinline__ int count_ge(uint4 (&buf)[kLoads], float cut) {
  constexpr int VE = Fmt<DT>::VE;
  const float c = fmaxf(cut, -kMaxFinite);  // -inf logits are never candidates
  fence_regs(buf);
  int n = 0;
#pragma unroll
  for (int i = 0; i < kLoads; ++i)
#pragma unroll
    for (int k = 0; k < VE; ++k) n += __popcll(__ballot(elem<DT>(buf[i], k) >= c));
  return n;
}

// Per-lane bitmask of the vectors holding an element >= cut.
template <int DT>
__device__ __forceinline__ uint32_t vectors_ge(uint4 (&buf)[kLoads], float cut) {
  constexpr int VE = Fmt<DT>::VE;
  const float c = fmaxf(cut, -kMaxFinite);
  fence_regs(buf);
  uint32_t mask = 0;
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    bool any = false;
#pragma unroll
    for (int k = 0; k < VE; ++k) any |= elem<DT>(buf[i], k) >= c;
    mask |= any ? (1u << i) : 0u;
  }
  return mask;
}

// Exact maximum of the chunk, and whether it holds a NaN or +inf.
template <int DT>
__device__ __forceinline__ float chunk_max(const uint4 (&buf)[kLoads], bool* bad) {
  constexpr int VE = Fmt<DT>::VE;
  float mx = -kInf;
  int nf = 0;
#pragma unroll
  for (int i = 0; i < kLoads; ++i)
#pragma unroll
    for (int k = 0; k < VE; ++k) {
      const float x = elem<DT>(buf[i], k);
      mx = fmaxf(mx, x);
      nf |= !(x < kInf);
    }
  *bad = __ballot(nf) != 0;
  return wave_max(mx);
}

// Top-k window: a cut whose candidate count lies in [need, cap].  Grows the
// window below the chunk max from d (logit units) until `need` tokens are in,
// then bisects while the list would overflow.  +inf when none exists.
template <int DT>
__device__ __forceinline__ float choose_cut(uint4 (&buf)[kLoads], float mx, float d, int need, int cap) {
  float lo = 0.0f;  // window known to hold < need tokens (or 0)
  float cut = mx - d;
  int n = count_ge<DT>(buf, cut);
  for (int it = 0; n < need && it < 64; ++it) {
    lo = d;
    d *= 4.0f;
    cut = mx - d;
    if (!(cut > -kMaxFinite)) {  // the window covers every finite logit
      cut = -kInf;
      n = count_ge<DT>(buf, cut);
      break;
    }
    n = count_ge<DT>(buf, cut);
  }
  if (n <= cap) return cut;
  float hi = d;
  for (int it = 0; it < 40; ++it) {
    const float mid = 0.5f * (lo + hi);
    if (!(mid > lo && mid < hi)) break;
    const float cm = mx - mid;
    const int nm = count_ge<DT>(buf, cm);
    if (nm < need) lo = mid;
    else if (nm > cap) hi = mid;
    else return cm;
  }
  return kInf;
}

// One exp per logit: returns the lane's sum of the terms 2^(x c2 - o) and
// the largest term of each of its vectors (emax[i]).  With o = r c2 rounded
// to fp32 each term is 2^((x - r) c2 + delta), delta = r c2 - o being common
// to all of them; the exponent x c2 - o is rounded once (fma).  The logits
// are only used through the terms, so each vector is unpacked right where
// it is consumed.
template <int DT>
__device__ __forceinline__ float exp_pass(const uint4 (&buf)[kLoads], float c2, float o, float (&emax)[kLoads]) {
  constexpr int VE = Fmt<DT>::VE;
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    float e[VE];
#pragma unroll
    for (int k = 0; k < VE; ++k) e[k] = __builtin_amdgcn_exp2f(fmaf(elem<DT>(buf[i], k), c2, -o));
    float si, mi;
    if constexpr (VE == 8) {
      si = ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
      mi = fmaxf(fmaxf(fmaxf(e[0], e[1]), e[2]), fmaxf(fmaxf(e[3], e[4]), e[5]));
      mi = fmaxf(fmaxf(mi, e[6]), e[7]);
    } else {
      si = (e[0] + e[1]) + (e[2] + e[3]);
      mi = fmaxf(fmaxf(fmaxf(e[0], e[1]), e[2]), e[3]);
    }
    emax[i] = mi;
    acc += si;
  }
  return acc;
}

// Lists the vectors flagged in `mask` (whole, from the registers) with the
// index of their first logit, in (vector, lane) order; returns how many
// there are (entries beyond cap are dropped).
__device__ __forceinline__ int list_vectors(uint4* dv, int32_t* di, uint32_t mask, const uint4 (&buf)[kLoads],
                                            int c0, int ve, int cap, int lane) {
  const uint64_t below = (1ull << lane) - 1ull;
  int n = 0;
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const bool h = (mask >> i) & 1u;
    const uint64_t bal = __ballot(h);
    if (h) {
      const int pos = n + __popcll(bal & below);
      if (pos < cap) {
        dv[pos] = buf[i];
        di[pos] = c0 + (i * kWave + lane) * ve;
      }
    }
    n += __popcll(bal);
  }
  return n;
}

// Softmax statistics of a plain / nucleus chunk from one exp per logit.
struct PlainStats {
  float o;        // exponent offset: terms are 2^(x c2 - o)
  double zw;      // sum of the chunk's terms
  double ma;      // the chunk maximum, from its largest term
  int st;         // 0 = statistics valid, 1 = no finite logit, 2 = NaN or +inf
  float emax[kLoads];  // largest term of each of the lane's vectors
};

// The exponent reference r is the largest logit of the lanes' first
// vectors.  A chunk whose terms overflow (a logit far above r) or hold a NaN
// is re-read once and redone from its exact maximum.
template <int DT, bool VEC>
__device__ __forceinline__ void plain_stats(uint4 (&buf)[kLoads], float c2, const char* row, int c0, int c1,
                                            int lane, PlainStats& ps) {
  constexpr int VE = Fmt<DT>::VE;
  float r = -kInf;
#pragma unroll
  for (int k = 0; k < VE; ++k) r = fmaxf(r, elem<DT>(buf[0], k));
  r = wave_max(r);
  float o = r * c2;
  float zt = 0.0f;
  const bool ok = r > -kInf && r < kInf;  // false on NaN
  if (ok) zt = exp_pass<DT>(buf, c2, o, ps.emax);
  ps.st = 0;
  if (!ok || __ballot(!(zt < kInf))) {
    // rare: re-read the chunk
    load_chunk<DT, VEC>(buf, row, c0, c1, lane);
    bool bad;
    const float mx = chunk_max<DT>(buf, &bad);
    ps.st = bad ? 2 : (mx == -kInf ? 1 : 0);
    o = mx * c2;
    zt = 0.0f;
    if (ps.st == 0) zt = exp_pass<DT>(buf, c2, o, ps.emax);  // every term <= 2^delta now
    else {
#pragma unroll
      for (int i = 0; i < kLoads; ++i) ps.emax[i] = 0.0f;
    }
  }
  float em = 0.0f;
#pragma unroll
  for (int i = 0; i < kLoads; ++i) em = fmaxf(em, ps.emax[i]);
  em = wave_max(em);
  ps.o = o;
  ps.zw = wave_sum((double)zt);
  // the largest term 2^a belongs to the chunk maximum x = (a + o) / c2
  ps.ma = ps.st == 0 ? ((double)log2f(em) + (double)o) / (double)c2 : -1e300;
}

// Finishes a plain / nucleus chunk.  A nucleus chunk lists every logit
// x >= g - 10/c2, where g >= the chunk maximum is the largest maximum among
// the chunks of the same row in this work-group (lists that overflow are
// retried with 8 and 6); its vectors are flagged from their largest terms
// with a 2^-8 margin in the exponent, a superset of those holding one.
template <int DT>
__device__ __forceinline__ void plain_finish(const KParams& P, const PlainStats& ps, float c2, bool cand,
                                             double g, const uint4 (&buf)[kLoads], size_t slot, int c0, int lane,
                                             ChunkRec& rec) {
  if (ps.st == 2) {
    rec.flags |= kCfNonFinite;
    return;
  }
  if (ps.st == 1) {
    rec.m = -kInf;
    rec.cut = -kInf;  // nothing finite: the (empty) candidate list is complete
    return;
  }
  const float m = (float)ps.ma;
  rec.m = m;
  // refer the sum to m: 2^(x c2 - o) = 2^((x - m) c2) 2^(m c2 - o)
  rec.z = ps.zw * exp2((double)ps.o - (double)m * (double)c2);
  if (cand) {
    uint4* dv = P.cvec + slot * (size_t)P.cap;
    int32_t* di = P.cidx + slot * (size_t)P.cap;
    int n = 0;
    float cut = kInf;
    for (int attempt = 0; attempt < 3; ++attempt) {
      cut = (float)(g - (attempt == 0 ? kCandLog2 : attempt == 1 ? 8.0f : 6.0f) / (double)c2);
      // x >= cut implies a term >= 2^(cut c2 - o) up to roundings far below the margin
      const float thr = exp2f((float)((double)cut * (double)c2 - (double)ps.o) - 0.00390625f);
      uint32_t mask = 0;
#pragma unroll
      for (int i = 0; i < kLoads; ++i) mask |= ps.emax[i] >= thr ? (1u << i) : 0u;
      n = list_vectors(dv, di, mask, buf, c0, Fmt<DT>::VE, P.cap, lane);
      if (n <= P.cap) break;
    }
    rec.cnt = n <= P.cap ? n : 0;
    rec.cut = n <= P.cap ? cut : kInf;  // +inf: incomplete, the merge falls back to the full row
  }
}

// Streaming pass: one wave per chunk.  The instance for MODE handles the
// sequences whose sampling mode is MODE; those whose effective mode is plain
// (top-p >= 1, top-k >= V) take the plain path.
template <int DT, bool VEC, int MODE>
__global__ __launch_bounds__(kThreads) void chunk_kernel(const KParams P) {
  constexpr int VE = Fmt<DT>::VE;
  constexpr int kWaves = kThreads / kWave;
  __shared__ float s_max[kWaves];
  __shared__ int s_key[kWaves];
  const int lane = (int)__lane_id();
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  const int S = P.S, R = P.R;
  const uint32_t gw = blockIdx.x * (uint32_t)kWaves + (uint32_t)wv;
  const int b = P.b_base + (int)(gw / (uint32_t)(R * S));
  const int rem = (int)(gw % (uint32_t)(R * S));
  const int r = rem / S, c = rem % S;
  // no early return: the nucleus instance meets at one barrier
  bool active = b < P.b_end && raw_mode(P, b) == MODE;
  SeqParams sp{};
  if (active) {
    sp = load_params(P, b);
    active = sp.valid;
  }
  bool tgt = false;
  int t = 0;
  if (active) active = decode_row(P, sp, r, &tgt, &t);  // padding rows are never read
  const char* row = active ? static_cast<const char*>(row_ptr<DT>(P, b, tgt, t)) : nullptr;
  const size_t slot = ((size_t)b * R + r) * S + c;
  const int c0 = c * P.L;
  const int c1 = min(P.V, c0 + P.L);
  const float c2 = (float)sp.c2;
  ChunkRec rec;
  rec.m = -kInf;
  rec.cut = kInf;
  rec.z = 0.0;
  rec.cnt = 0;
  rec.arg = -1;
  rec.flags = 0;
  rec.pad = 0;
  uint4 buf[kLoads];
  if (active) load_chunk<DT, VEC>(buf, row, c0, c1, lane);

  const bool special = active && (MODE == SV_TOPK || MODE == SV_GREEDY) && sp.mode == MODE;
  if (special) {
    bool bad;
    const float mx = chunk_max<DT>(buf, &bad);
    rec.m = mx;
    if (bad) {
      rec.flags |= kCfNonFinite;
    } else if (MODE == SV_GREEDY) {
      int best = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < kLoads; ++i)
#pragma unroll
        for (int k = 0; k < VE; ++k)
          if (elem<DT>(buf[i], k) == mx) best = min(best, c0 + (i * kWave + lane) * VE + k);
      rec.arg = wave_min_i(best);
    } else {
      const int need = sp.topk, cap = P.cap;
      float cut = kInf;
      if (need <= cap) cut = choose_cut<DT>(buf, mx, 2.0f, need, cap);
      if (cut != kInf) {
        const int n = list_vectors(P.cvec + slot * (size_t)cap, P.cidx + slot * (size_t)cap,
                                   vectors_ge<DT>(buf, cut), buf, c0, VE, cap, lane);
        rec.cnt = min(n, cap);
        rec.cut = n <= cap ? cut : kInf;
      }
    }
  }
  if constexpr (MODE != SV_GREEDY) {
    const bool plain = active && !special;
    const bool cand = plain && MODE == SV_TOPP && sp.mode == SV_TOPP;
    PlainStats ps;
    ps.st = 1;
    ps.ma = -1e300;
    if (plain) plain_stats<DT, VEC>(buf, c2, row, c0, c1, lane, ps);
    double g = ps.ma;
    if constexpr (MODE == SV_TOPP) {
      // the largest chunk maximum among this work-group's chunks of the same row
      if (lane == 0) {
        s_key[wv] = cand ? (int)(gw / (uint32_t)S) : -1;
        s_max[wv] = ps.st == 0 ? (float)ps.ma : -kInf;
      }
      __syncthreads();
      const int key = cand ? (int)(gw / (uint32_t)S) : -2;
#pragma unroll
      for (int w = 0; w < kWaves; ++w)
        if (s_key[w] == key) g = fmax(g, (double)s_max[w]);
    }
    if (plain) plain_finish<DT>(P, ps, c2, cand, g, buf, slot, c0, lane, rec);
  }
  if (active && lane == 0) P.chunks[slot] = rec;
}

// ======================================================= merge kernel ====

struct SmemMerge {
  int pre[kMaxChunks];  // first flat candidate index of each chunk
  float cx[kMergeCache];
  int cidx[kMergeCache];
  unsigned long long cm[kMergeCache];
  uint32_t hc[256];
  unsigned long long hm[256];
  alignas(16) int kidx[kListMax + 4];
  unsigned long long km[kListMax];
  int n, nk;
  uint32_t sel_digit, sel_hit;
  Red red;
};

struct SelOut {
  float T;
  bool reached;
  uint32_t n_keep;
  unsigned long long m_keep, m_above;
};

// MSB-first radix selection over order-preserving keys.  Finds the largest
// logit value T whose inclusive descending cumulative count (top-k) or mass
// (nucleus, fixed point) reaches `target`.  Histograms hold counts and
// fixed-point masses, so the result does not depend on atomic order.
// `each(f)` calls f(x, mass) for this thread's share of the elements.
template <int DT, class Each>
__device__ __forceinline__ SelOut radix_select(Each&& each, bool by_mass, unsigned long long target,
                                               SmemMerge& sm) {
  const int tid = threadIdx.x;
  const int levels = DT == SV_BF16 ? 2 : 4;
  uint32_t pkey = 0, pmask = 0;
  unsigned long long above_c = 0, above_m = 0;
  bool reached = true;
  unsigned long long last_c = 0, last_m = 0;
  for (int lv = 0; lv < levels; ++lv) {
    const int shift = 24 - 8 * lv;
    __syncthreads();
    sm.hc[tid] = 0;
    sm.hm[tid] = 0;
    __syncthreads();
    each([&](float x, unsigned long long m) {
      const uint32_t key = fkey(x);
      if ((key & pmask) == pkey) {
        const uint32_t dg = (key >> shift) & 255u;
        atomicAdd(&sm.hc[dg], 1u);
        atomicAdd(&sm.hm[dg], m);
      }
    });
    __syncthreads();
    if (tid < 64) {
      // lane l owns digits 4l..4l+3; suffix sums run from digit 255 down
      const int lane = tid;
      unsigned long long c[4], m[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = sm.hc[4 * lane + j];
        m[j] = sm.hm[4 * lane + j];
      }
      const unsigned long long lc = c[0] + c[1] + c[2] + c[3];
      const unsigned long long lm = m[0] + m[1] + m[2] + m[3];
      unsigned long long sc = lc, sms = lm;  // inclusive suffix over lanes >= lane
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const unsigned long long yc = __shfl_down(sc, o);
        const unsigned long long ym = __shfl_down(sms, o);
        if (lane + o < 64) {
          sc += yc;
          sms += ym;
        }
      }
      unsigned long long rc = sc - lc, rm = sms - lm;  // digits of higher lanes
      int best = -1;
#pragma unroll
      for (int j = 3; j >= 0; --j) {
        rc += c[j];
        rm += m[j];
        const bool ok = by_mass ? (above_m + rm >= target) : (above_c + rc >= target);
        if (ok && best < 0) best = 4 * lane + j;
      }
      const int hit = wave_max_i(best);
      int lowest = 256;
#pragma unroll
      for (int j = 3; j >= 0; --j)
        if (c[j] > 0) lowest = 4 * lane + j;
      const int low = wave_min_i(lowest);
      if (lane == 0) {
        sm.sel_hit = hit >= 0 ? 1u : 0u;
        sm.sel_digit = hit >= 0 ? (uint32_t)hit : (low < 256 ? (uint32_t)low : 0u);
      }
    }
    __syncthreads();
    const uint32_t dg = sm.sel_digit;
    if (!sm.sel_hit) reached = false;
    // everything strictly above the chosen digit joins the "above" totals
    const unsigned long long add_c = block_sum_u64((int)tid > (int)dg ? sm.hc[tid] : 0ull, sm.red);
    const unsigned long long add_m = block_sum_u64((int)tid > (int)dg ? sm.hm[tid] : 0ull, sm.red);
    above_c += add_c;
    above_m += add_m;
    last_c = sm.hc[dg];
    last_m = sm.hm[dg];
    pkey |= dg << shift;
    pmask |= 255u << shift;
  }
  if (DT == SV_BF16) pkey |= (pkey >> 31) ? 0u : 0xFFFFu;
  SelOut r;
  r.T = key_value(pkey);
  r.reached = reached;
  r.n_keep = (uint32_t)(above_c + last_c);
  r.m_keep = above_m + last_m;
  r.m_above = above_m;
  return r;
}

__device__ __forceinline__ unsigned long long fixed_mass(double e) {
  return (unsigned long long)(e * kFix + 0.5);
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void merge_kernel(const KParams P) {
  __shared__ SmemMerge sm;
  const int tid = threadIdx.x;
  const int S = P.S, R = P.R;
  const uint32_t blk = blockIdx.x;
  const int b = P.b_base + (int)(blk / (uint32_t)R);
  const int r = (int)(blk % (uint32_t)R);
  const SeqParams sp = load_params(P, b);
  if (!sp.valid) return;
  bool tgt;
  int t;
  if (!decode_row(P, sp, r, &tgt, &t)) return;
  const void* row = row_ptr<DT>(P, b, tgt, t);
  const size_t rowid = (size_t)b * R + r;
  const size_t slot0 = rowid * S;
  const int mode = sp.mode;
  const int tok = t < sp.Kb ? P.tokens[(size_t)b * P.K_max + t] : INT32_MIN;

  const ChunkRec* crec = P.chunks + slot0;
  float m_s = -kInf;
  int f_s = 0;
  for (int s = tid; s < S; s += kThreads) {
    m_s = fmaxf(m_s, crec[s].m);
    f_s |= (int)crec[s].flags;
  }
  const float M = block_max(m_s, sm.red);
  const int cflags = block_max_i(f_s, sm.red);

  RowRec rr;
  rr.M = M;
  rr.T = -kInf;
  rr.c2 = sp.c2;
  rr.Zs = 1.0;
  rr.pid = __builtin_nan("");
  rr.g = -1;
  rr.n_keep = -1;
  rr.flags = 0;
  rr.pad = 0;
  if ((cflags & kCfNonFinite) || !(M < kInf) || isnan(M)) rr.flags |= SV_ST_NONFINITE;
  else if (M == -kInf) rr.flags |= SV_ST_EMPTY;

  double Z = 0.0;
  if (!(rr.flags & kErrBits) && (mode == SV_PLAIN || mode == SV_TOPP)) {
    double term = 0.0;
    for (int s = tid; s < S; s += kThreads) {
      const ChunkRec c = crec[s];
      if (c.m > -kInf) term += c.z * exp2(((double)c.m - (double)M) * sp.c2);
    }
    Z = block_sum(term, sm.red);
    if (!(Z > 0.0) || !(Z < 1e300)) rr.flags |= SV_ST_NONFINITE;
  }

  bool list_kept = false;
  if (!(rr.flags & kErrBits)) {
    if (mode == SV_PLAIN) {
      rr.Zs = Z;
    } else if (mode == SV_GREEDY) {
      int best = 0x7fffffff;
      for (int s = tid; s < S; s += kThreads)
        if (crec[s].m == M) best = min(best, crec[s].arg);
      rr.g = block_min_i(best, sm.red);
      rr.T = M;
      rr.n_keep = 1;
    } else {
      // candidates >= C, where C = max over chunks of the chunk cuts: every
      // logit >= C of the row is among them
      float cmax = -kInf;
      for (int s = tid; s < S; s += kThreads) cmax = fmaxf(cmax, crec[s].cut);
      const float C = block_max(cmax, sm.red);
      const bool by_mass = mode == SV_TOPP;
      unsigned long long target;
      if (by_mass) {
        const double tt = (double)sp.topp * Z * kFix;
        target = tt < 1.0 ? 1ull : (unsigned long long)tt;
      } else {
        target = (unsigned long long)sp.topk;
      }
      bool fast = C < kInf;
      if (fast) {
        // one flat index over the chunks' lists: thread t counts chunks 4t..4t+3
        int cn[4], ls = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int s = 4 * tid + q;
          cn[q] = s < S ? crec[s].cnt : 0;
          ls += cn[q];
        }
        double tot;
        int run = (int)block_exclusive_scan((double)ls, &tot, sm.red);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (4 * tid + q < S) sm.pre[4 * tid + q] = run;
          run += cn[q];
        }
        if (tid == 0) sm.n = 0;
        __syncthreads();
        const int total = (int)tot;
        const float Cf = fmaxf(C, -kMaxFinite);
        for (int f = tid; f < total; f += kThreads) {
          int lo = 0, hi = S - 1;  // the last chunk whose list starts at or before f
          while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (sm.pre[mid] <= f) lo = mid;
            else hi = mid - 1;
          }
          const size_t at = (slot0 + lo) * (size_t)P.cap + (f - sm.pre[lo]);
          const uint4 v = P.cvec[at];
          const int e0 = P.cidx[at];
#pragma unroll
          for (int k = 0; k < Fmt<DT>::VE; ++k) {
            const float x = elem<DT>(v, k);
            if (x >= Cf) {  // -inf padding past the row end never passes
              const int pos = atomicAdd(&sm.n, 1);
              if (pos < kMergeCache) {
                sm.cx[pos] = x;
                sm.cidx[pos] = e0 + k;
                sm.cm[pos] = fixed_mass(exp2(((double)x - (double)M) * sp.c2));
              }
            }
          }
        }
        __syncthreads();
        fast = sm.n <= kMergeCache;
      }
      SelOut so;
      if (fast) {
        const int n = sm.n;
        so = radix_select<DT>(
            [&](auto&& f) {
              for (int j = tid; j < n; j += kThreads) f(sm.cx[j], sm.cm[j]);
            },
            by_mass, target, sm);
        fast = so.reached && so.T >= C;
      }
      if (!fast) {
        // full-row selection: re-read the row (rare: an incomplete or
        // insufficient candidate window)
        const float c2f = (float)sp.c2;
        so = radix_select<DT>(
            [&](auto&& f) {
              for (int e = tid; e < P.V; e += kThreads) {
                const float x = load_logit<DT>(row, e);
                f(x, fixed_mass((double)__builtin_amdgcn_exp2f((x - M) * c2f)));
              }
            },
            by_mass, target, sm);
        rr.flags |= SV_ST_FULLSELECT;
      }
      rr.T = so.T;
      rr.n_keep = (int)so.n_keep;
      rr.Zs = (double)so.m_keep / kFix;
      if (by_mass) {
        const double lo = (double)so.m_above / kFix / Z, hi = (double)so.m_keep / kFix / Z;
        if (fabs(lo - (double)sp.topp) < kWindow || fabs(hi - (double)sp.topp) < kWindow)
          rr.flags |= SV_ST_MARGIN;
      }
      if (!(rr.Zs > 0.0)) rr.flags |= SV_ST_EMPTY;
      list_kept = fast && tgt && so.n_keep <= (uint32_t)kListMax;
    }
  }

  if (tok != INT32_MIN) {  // this row scores a draft token
    if (tok < 0 || tok >= P.V) {
      rr.flags |= SV_ST_TOKEN;
    } else if (!(rr.flags & kErrBits)) {
      if (mode == SV_GREEDY) {
        rr.pid = tok == rr.g ? 1.0 : 0.0;
      } else {
        const float x = load_logit<DT>(row, tok);
        rr.pid = x >= rr.T ? exp2(((double)x - (double)M) * sp.c2) / rr.Zs : 0.0;
      }
    }
  }

  if (list_kept && !(rr.flags & kErrBits)) {
    // the target row's kept set, in vocabulary order, with probabilities:
    // compact it, then rank each entry by its vocabulary index
    rr.flags |= kRfListOk;
    const int n = sm.n;
    __syncthreads();
    if (tid == 0) sm.nk = 0;
    __syncthreads();
    for (int j = tid; j < n; j += kThreads) {
      if (sm.cx[j] >= rr.T) {
        const int pos = atomicAdd(&sm.nk, 1);
        sm.kidx[pos] = sm.cidx[j];
        sm.km[pos] = sm.cm[j];
      }
    }
    __syncthreads();
    const int nk = sm.nk;  // == n_keep <= kListMax
    for (int j = nk; j < ((nk + 3) & ~3); ++j)
      if (tid == 0) sm.kidx[j] = 0x7fffffff;  // pad to whole int4s
    __syncthreads();
    KeptEntry* out = P.kept + rowid * kListMax;
    const int4* k4 = reinterpret_cast<const int4*>(sm.kidx);
    for (int j = tid; j < nk; j += kThreads) {
      const int my = sm.kidx[j];
      int rank = 0;
      for (int i = 0; i < (nk + 3) / 4; ++i) {
        const int4 v = k4[i];
        rank += (v.x < my) + (v.y < my) + (v.z < my) + (v.w < my);
      }
      KeptEntry ke;
      ke.idx = my;
      ke.pad = 0;
      ke.q = (double)sm.km[j] / kFix / rr.Zs;
      out[rank] = ke;
    }
  }
  if (tid == 0) P.rows[rowid] = rr;
}

// ======================================================= final kernel ====

struct SmemFinal {
  int idx[kListMax];
  double w[kListMax];
  double c[kListMax];
  Red red;
  uint32_t misc[4];
};

struct Draw {
  int y;
  double S;
  uint32_t flags;
};

// Inverse CDF over the target's kept set (vocabulary order): w = (q - p)+
// when resampling, else w = q.
template <int DT>
__device__ __forceinline__ Draw draw_from_list(const KParams& P, const RowRec& rq, bool resample,
                                               const RowRec& rp, size_t rowq, const void* drow, double u,
                                               SmemFinal& sm) {
  const int tid = threadIdx.x;
  const int N = rq.n_keep;  // <= kListMax
  const KeptEntry* kl = P.kept + rowq * kListMax;
  double qv[2];
  int iv[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int i = 2 * tid + j;
    qv[j] = 0.0;
    iv[j] = 0;
    if (i < N) {
      const KeptEntry ke = kl[i];
      qv[j] = ke.q;
      iv[j] = ke.idx;
    }
  }
  Draw d;
  d.flags = 0;
  double w[2];
  bool use_p = resample;
  double total = 0.0, ex = 0.0;
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      w[j] = qv[j];
      if (use_p && 2 * tid + j < N) {
        const float xp = load_logit<DT>(drow, iv[j]);
        const double p = xp >= rp.T ? exp2(((double)xp - (double)rp.M) * rp.c2) / rp.Zs : 0.0;
        w[j] = qv[j] > p ? qv[j] - p : 0.0;
      }
    }
    ex = block_exclusive_scan(w[0] + w[1], &total, sm.red);
    if (total > 0.0 || !use_p) break;
    d.flags |= SV_ST_ZERO_RESIDUAL;  // (q - p)+ has no mass: draw from q
    use_p = false;
  }
  d.S = total;
  const double target = u * total;
  // first element whose running sum exceeds the target; last non-zero one
  int first = 0x7fffffff, lastnz = -1, firstnz = 0x7fffffff;
  double c = ex;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int i = 2 * tid + j;
    const double cn = c + w[j];
    if (i < N) {
      sm.w[i] = w[j];
      sm.c[i] = cn;
      sm.idx[i] = iv[j];
      if (w[j] > 0.0) {
        if (cn > target) first = min(first, i);
        lastnz = max(lastnz, i);
        firstnz = min(firstnz, i);
      }
    }
    c = cn;
  }
  first = block_min_i(first, sm.red);
  lastnz = block_max_i(lastnz, sm.red);
  firstnz = block_min_i(firstnz, sm.red);
  int iy = first <= lastnz ? first : lastnz;
  if (iy < 0) iy = 0;
  d.y = N > 0 ? sm.idx[iy] : 0;
  if (N > 0 && lastnz >= 0) {
    // margins of interior CDF boundaries
    const double hi = sm.c[iy] / d.S, lo = (sm.c[iy] - sm.w[iy]) / d.S;
    if ((firstnz < iy && u - lo < kWindow) || (lastnz > iy && hi - u < kWindow)) d.flags |= SV_ST_MARGIN;
  }
  return d;
}

template <int DT>
__device__ __forceinline__ double weight(const RowRec& rq, bool use_p, const RowRec& rp, float xq, float xp) {
  double q = 0.0;
  if (xq >= rq.T) q = (double)__builtin_amdgcn_exp2f((xq - rq.M) * (float)rq.c2) / rq.Zs;
  if (!use_p) return q;
  double p = 0.0;
  if (xp >= rp.T) p = (double)__builtin_amdgcn_exp2f((xp - rp.M) * (float)rp.c2) / rp.Zs;
  return q > p ? q - p : 0.0;
}

// Inverse CDF over full logit rows re-read from memory, in tiles of
// 256 x 8 tokens (thread t owns tokens 8t..8t+7 of a tile).
template <int DT>
__device__ __forceinline__ Draw draw_from_rows(const KParams& P, const RowRec& rq, bool resample,
                                               const RowRec& rp, const void* qrow, const void* prow,
                                               double u, SmemFinal& sm) {
  const int tid = threadIdx.x;
  const int V = P.V;
  constexpr int TILE = kThreads * 8;
  Draw d;
  d.flags = SV_ST_REREAD;
  d.y = 0;
  d.S = 0.0;
  bool use_p = resample;
  for (int pass = 0; pass < 2; ++pass) {
    // total mass and the first / last token of non-zero weight
    double S = 0.0;
    int nz_lo = 0x7fffffff, nz_hi = -1;
    for (int base = 0; base < V; base += TILE) {
      double s = 0.0;
      for (int k = 0; k < 8; ++k) {
        const int e = base + 8 * tid + k;
        if (e < V) {
          const double w = weight<DT>(rq, use_p, rp, load_logit<DT>(qrow, e), use_p ? load_logit<DT>(prow, e) : 0.f);
          s += w;
          if (w > 0.0) {
            nz_lo = min(nz_lo, e);
            nz_hi = max(nz_hi, e);
          }
        }
      }
      S += block_sum(s, sm.red);
    }
    nz_lo = block_min_i(nz_lo, sm.red);
    nz_hi = block_max_i(nz_hi, sm.red);
    if (!(S > 0.0) && pass == 0 && use_p) {
      d.flags |= SV_ST_ZERO_RESIDUAL;
      use_p = false;
      continue;
    }
    d.S = S;
    const double target = u * S;
    double run = 0.0;
    int y = -1;
    double lo = 0.0, hi = 0.0;
    for (int base = 0; base < V && y < 0; base += TILE) {
      double wk[8];
      double s = 0.0;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int e = base + 8 * tid + k;
        wk[k] = e < V ? weight<DT>(rq, use_p, rp, load_logit<DT>(qrow, e), use_p ? load_logit<DT>(prow, e) : 0.f) : 0.0;
        s += wk[k];
      }
      double tile;
      const double ex = block_exclusive_scan(s, &tile, sm.red);
      if (run + tile > target) {
        // the thread whose span crosses the target finds the token
        int cand = 0x7fffffff;
        double c = run + ex;
        double cl = 0.0, ch = 0.0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const double cn = c + wk[k];
          if (cn > target && wk[k] > 0.0 && cand == 0x7fffffff) {
            cand = base + 8 * tid + k;
            cl = c;
            ch = cn;
          }
          c = cn;
        }
        const int ymin = block_min_i(cand, sm.red);
        if (ymin != 0x7fffffff) {
          if (cand == ymin) {
            sm.red.d[0] = cl;  // block_min_i has returned: its slots are free
            sm.red.d[1] = ch;
          }
          __syncthreads();
          lo = sm.red.d[0];
          hi = sm.red.d[1];
          __syncthreads();
          y = ymin;
        }
      }
      run += tile;
    }
    if (y < 0) {  // rounding left no token above the target
      y = nz_hi < 0 ? 0 : nz_hi;
      lo = S;
      hi = S;
    }
    d.y = y;
    if (nz_lo < y && u - lo / S < kWindow) d.flags |= SV_ST_MARGIN;
    if (nz_hi > y && hi / S - u < kWindow) d.flags |= SV_ST_MARGIN;
    break;
  }
  return d;
}

__device__ __forceinline__ void write_error(const KParams& P, int b, uint32_t st) {
  const int tid = threadIdx.x;
  for (int i = tid; i <= P.K_max; i += kThreads) P.out_tokens[(size_t)b * (P.K_max + 1) + i] = -1;
  if (P.diag)
    for (int i = tid; i < 2 * P.K_max; i += kThreads) P.diag[(size_t)b * 2 * P.K_max + i] = __builtin_nanf("");
  if (tid == 0) {
    P.accepted[b] = -1;
    if (P.status) P.status[b] = st;
  }
}

template <int DT>
__global__ __launch_bounds__(kThreads) void final_kernel(const KParams P) {
  __shared__ SmemFinal sm;
  const int tid = threadIdx.x;
  const int b = P.b_base + (int)blockIdx.x;
  const SeqParams sp = load_params(P, b);
  if (!sp.valid) {
    write_error(P, b, SV_ST_PARAM);
    return;
  }
  const int Kb = sp.Kb, KM = P.K_max, R = P.R;
  const uint64_t g = P.row_offset + (uint64_t)b;
  const size_t rbase = (size_t)b * R;

  // OR of the used rows' flags
  uint32_t v = 0;
  for (int t = tid; t <= Kb; t += kThreads) v |= P.rows[rbase + t].flags;
  for (int t = tid; t < Kb; t += kThreads) v |= P.rows[rbase + KM + 1 + t].flags;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v |= (uint32_t)__shfl_xor((int)v, o);
  __syncthreads();
  if ((tid & 63) == 0) sm.red.i[tid >> 6] = (int)v;
  __syncthreads();
  uint32_t st = (uint32_t)(sm.red.i[0] | sm.red.i[1] | sm.red.i[2] | sm.red.i[3]);
  __syncthreads();
  st &= ~kRfListOk;
  if (st & kErrBits) {
    write_error(P, b, st & kErrBits);
    return;
  }
  // accept walk (one thread; K_b <= 64)
  if (tid == 0) {
    int n = Kb;
    uint32_t s2 = 0;
    for (int t = 0; t < Kb; ++t) {
      const double q = P.rows[rbase + t].pid, p = P.rows[rbase + KM + 1 + t].pid;
      if (P.diag) {
        P.diag[((size_t)b * KM + t) * 2 + 0] = (float)q;
        P.diag[((size_t)b * KM + t) * 2 + 1] = (float)p;
      }
      if (n < Kb) continue;
      const double u = uniform24(P.seed, g, (uint32_t)t, kPurposeAccept);
      if (p == 0.0) s2 |= SV_ST_PZERO;
      const bool accept = u * p < q;
      if (p > 0.0) {
        const double ratio = q / p;
        if (ratio < 1.0 + kWindow && fabs(u - ratio) < kWindow) s2 |= SV_ST_MARGIN;
      }
      if (!accept) n = t;
    }
    if (P.diag)
      for (int t = Kb; t < KM; ++t) {
        P.diag[((size_t)b * KM + t) * 2 + 0] = __builtin_nanf("");
        P.diag[((size_t)b * KM + t) * 2 + 1] = __builtin_nanf("");
      }
    sm.misc[0] = (uint32_t)n;
    sm.misc[1] = s2;
  }
  __syncthreads();
  const int n = (int)sm.misc[0];
  st |= sm.misc[1];
  __syncthreads();

  const bool resample = n < Kb;
  const RowRec rq = P.rows[rbase + n];
  RowRec rp = rq;
  if (resample) rp = P.rows[rbase + KM + 1 + n];
  const double u = uniform24(P.seed, g, (uint32_t)n, resample ? kPurposeResample : kPurposeBonus);
  Draw d;
  if (sp.mode == SV_GREEDY) {
    d.y = rq.g;
    d.S = 1.0;
    d.flags = (resample && rp.g == rq.g) ? SV_ST_ZERO_RESIDUAL : 0u;
  } else if (rq.flags & kRfListOk) {
    d = draw_from_list<DT>(P, rq, resample, rp, rbase + n, resample ? row_ptr<DT>(P, b, false, n) : nullptr,
                           u, sm);
  } else {
    d = draw_from_rows<DT>(P, rq, resample, rp, row_ptr<DT>(P, b, true, n),
                           resample ? row_ptr<DT>(P, b, false, n) : nullptr, u, sm);
  }
  st |= d.flags;
  for (int i = tid; i <= KM; i += kThreads) {
    int val = -1;
    if (i < n) val = P.tokens[(size_t)b * KM + i];
    else if (i == n) val = d.y;
    P.out_tokens[(size_t)b * (KM + 1) + i] = val;
  }
  if (tid == 0) {
    P.accepted[b] = n;
    if (P.status) P.status[b] = st & ~kRfListOk;
  }
}

template <int DT, bool VEC>
void launch_chunk(const KParams& p, int mode, dim3 grid, hipStream_t stream) {
  const dim3 block(kThreads);
  switch (mode) {
    case SV_PLAIN: hipLaunchKernelGGL((chunk_kernel<DT, VEC, SV_PLAIN>), grid, block, 0, stream, p); break;
    case SV_TOPK: hipLaunchKernelGGL((chunk_kernel<DT, VEC, SV_TOPK>), grid, block, 0, stream, p); break;
    case SV_TOPP: hipLaunchKernelGGL((chunk_kernel<DT, VEC, SV_TOPP>), grid, block, 0, stream, p); break;
    default: hipLaunchKernelGGL((chunk_kernel<DT, VEC, SV_GREEDY>), grid, block, 0, stream, p); break;
  }
}

template <int DT, bool VEC>
void launch_all(const KParams& p, int nseq, hipStream_t stream) {
  const dim3 block(kThreads);
  // one streaming instance per sampling mode that can occur
  for (int mode = SV_PLAIN; mode <= SV_GREEDY; ++mode) {
    if (!p.mode && mode != p.dmode) continue;
    const size_t waves = (size_t)nseq * p.R * p.S;
    launch_chunk<DT, VEC>(p, mode, dim3((unsigned)((waves + kThreads / kWave - 1) / (kThreads / kWave))), stream);
  }
  hipLaunchKernelGGL((merge_kernel<DT, VEC>), dim3((unsigned)((size_t)nseq * p.R)), block, 0, stream, p);
  hipLaunchKernelGGL((final_kernel<DT>), dim3((unsigned)nseq), block, 0, stream, p);
}

}  // namespace

hipError_t launch_verify(const KParams& p, int dtype, bool vec, int nseq, hipStream_t stream) {
  if (nseq <= 0) return hipSuccess;
  if (dtype == SV_BF16) {
    if (vec) launch_all<SV_BF16, true>(p, nseq, stream);
    else launch_all<SV_BF16, false>(p, nseq, stream);
  } else {
    if (vec) launch_all<SV_F32, true>(p, nseq, stream);
    else launch_all<SV_F32, false>(p, nseq, stream);
  }
  return hipGetLastError();
}

}  // namespace sv
