// gfx950 kernels of the verify-and-resample step of speculative sampling.
//
// One fused launch per call.  The grid is (sequence, logit row, chunk):
// every used logit row (target positions 0..K_b, draft positions 0..K_b-1)
// is split into S chunks of at most 32768 bf16 / 16384 fp32 logits, and each
// work-group streams one chunk from HBM into registers exactly once.  The
// work is chained without host round trips or extra launches:
//
//   chunk pass  (every WG)       max, sum of 2^((x - m) c2), nucleus / top-k
//                                candidates, greedy argmax -> ChunkRec
//   row merge   (last chunk WG   log-sum-exp merge, threshold selection,
//                of a row)       kept mass, probability of the draft token
//                                -> RowRec
//   finalize    (last row WG of  accept walk, first rejection, resample from
//                a sequence)     normalize((q - p)+) or bonus draw, outputs
//
// "Last" is decided with a device-scope counter per row and per sequence
// (release fence, atomic increment, acquire fence); no work-group ever waits
// for another, so there is no co-residency assumption.  The counters reset
// themselves, so a call needs no memset.
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
constexpr double kLog2e = 1.4426950408889634074;
// Fixed-point scale of masses (units of the row's largest term): integer
// accumulation makes histogram sums independent of atomic order.
constexpr double kFix = 1099511627776.0;  // 2^40
constexpr double kWindow = 1e-6;
// Nucleus candidates: tokens whose term is within 2^-12 of the chunk's
// largest term.
constexpr float kCandLog2 = 12.0f;

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
  float f[4];
  double d[4];
  int i[4];
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

__device__ __forceinline__ SeqParams load_params(const KParams& P, int b) {
  SeqParams s;
  s.Kb = P.kpr ? P.kpr[b] : P.K_max;
  s.mode = P.mode ? (int)P.mode[b] : P.dmode;
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

// --------------------------------------------------------- shared mem ----
struct SmemChunk {
  float2 cand[kCandCap];
  int cnt;
};
struct SmemMerge {
  ChunkRec crec[kMaxChunks];
  uint32_t hc[256];
  unsigned long long hm[256];
  uint32_t sel_digit;
  uint32_t sel_hit;
};
struct SmemFinal {
  float x[kListMax];
  int idx[kListMax];
  float sx[kListMax];
  int sidx[kListMax];
  double w[kListMax];
  double c[kListMax];
  int n;
};
struct Smem {
  union {
    SmemChunk ch;
    SmemMerge mg;
    SmemFinal fin;
  };
  Red red;
  int flag;
};

// ------------------------------------------------------- chunk pass -----
// Loads this thread's part of chunk [c0, c1) into registers: vector i holds
// logits c0 + (i * 256 + tid) * VE + [0, VE).  Every load is issued
// unconditionally from a clamped in-bounds address and the out-of-range
// vectors are replaced by -inf afterwards, so all kLoads requests are in
// flight together.
template <int DT, bool VEC>
__device__ __forceinline__ void load_chunk(uint4 (&buf)[kLoads], const char* row, int c0, int c1) {
  constexpr int VE = Fmt<DT>::VE, ES = Fmt<DT>::ES;
  const int tid = threadIdx.x;
  const uint32_t ninf = DT == SV_BF16 ? 0xff80ff80u : 0xff800000u;
  if constexpr (VEC) {
    // c0 and c1 are multiples of VE and c1 - c0 >= VE
    const int last = c1 - VE;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int e0 = c0 + (i * kThreads + tid) * VE;
      buf[i] = *reinterpret_cast<const uint4*>(row + (size_t)min(e0, last) * ES);
    }
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const bool ok = c0 + (i * kThreads + tid) * VE < c1;
      buf[i].x = ok ? buf[i].x : ninf;
      buf[i].y = ok ? buf[i].y : ninf;
      buf[i].z = ok ? buf[i].z : ninf;
      buf[i].w = ok ? buf[i].w : ninf;
    }
  } else {
    const int last = c1 - 1;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int e0 = c0 + (i * kThreads + tid) * VE;
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
// unpacks them again instead of keeping 128 unpacked values live (which would
// double the register footprint and spill).
__device__ __forceinline__ void fence_regs(uint4 (&buf)[kLoads]) {
#pragma unroll
  for (int i = 0; i < kLoads; ++i)
    asm volatile("" : "+v"(buf[i].x), "+v"(buf[i].y), "+v"(buf[i].z), "+v"(buf[i].w));
}

template <int DT>
__device__ __forceinline__ int count_ge(uint4 (&buf)[kLoads], float cut, Red& red) {
  constexpr int VE = Fmt<DT>::VE;
  // -inf logits are never candidates
  const float c = fmaxf(cut, -3.402823466e38f);
  fence_regs(buf);
  // wave-uniform count: compare into a lane mask, popcount on the scalar unit
  int n = 0;
#pragma unroll
  for (int i = 0; i < kLoads; ++i)
#pragma unroll
    for (int k = 0; k < VE; ++k) n += __popcll(__ballot(elem<DT>(buf[i], k) >= c));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red.i[threadIdx.x >> 6] = n;
  __syncthreads();
  return (red.i[0] + red.i[1]) + (red.i[2] + red.i[3]);
}

// Appends (logit, index) of this vector's elements >= c to the chunk list.
template <int DT>
__device__ __forceinline__ void append_vec(const uint4& v, float c, int e0, int cap, Smem& sm) {
  constexpr int VE = Fmt<DT>::VE;
#pragma unroll
  for (int k = 0; k < VE; ++k) {
    const float x = elem<DT>(v, k);
    if (x >= c) {
      const int pos = atomicAdd(&sm.ch.cnt, 1);
      if (pos < cap) sm.ch.cand[pos] = make_float2(x, __int_as_float(e0 + k));
    }
  }
}

template <int DT>
__device__ __forceinline__ void collect_ge(uint4 (&buf)[kLoads], float cut, int c0, int cap,
                                           Smem& sm) {
  constexpr int VE = Fmt<DT>::VE;
  const float c = fmaxf(cut, -3.402823466e38f);
  const int tid = threadIdx.x;
  fence_regs(buf);
  __syncthreads();
  if (tid == 0) sm.ch.cnt = 0;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    bool any = false;
#pragma unroll
    for (int k = 0; k < VE; ++k) any |= elem<DT>(buf[i], k) >= c;
    if (any) append_vec<DT>(buf[i], c, c0 + (i * kThreads + tid) * VE, cap, sm);
  }
  __syncthreads();
}

// Picks a cut such that the candidate count lies in [need, cap]; grows the
// window from `d` (raw logit units below the chunk max) until `need` tokens
// are in, then shrinks it while the list would overflow.  Returns +inf when
// no such cut exists (the list would be incomplete).
template <int DT>
__device__ __forceinline__ float choose_cut(uint4 (&buf)[kLoads], float mx, float d, int need, int cap, Red& red) {
  float lo = 0.0f;  // window known to hold < need tokens (or 0)
  float cut = mx - d;
  int n = count_ge<DT>(buf, cut, red);
  for (int it = 0; n < need && it < 64; ++it) {
    lo = d;
    d *= 4.0f;
    cut = mx - d;
    if (!(cut > -3.402823466e38f)) {  // window covers every finite logit
      cut = -kInf;
      n = count_ge<DT>(buf, cut, red);
      break;
    }
    n = count_ge<DT>(buf, cut, red);
  }
  if (n <= cap) return cut;
  float hi = d;
  for (int it = 0; it < 40; ++it) {
    const float mid = 0.5f * (lo + hi);
    if (!(mid > lo && mid < hi)) break;
    const float cm = mx - mid;
    const int nm = count_ge<DT>(buf, cm, red);
    if (nm < need) {
      lo = mid;
    } else if (nm > cap) {
      hi = mid;
    } else {
      return cm;
    }
  }
  return kInf;
}

// Counting and collecting straight from the chunk in memory (cache-resident
// after the streaming load); used only when a nucleus window overflows the
// candidate list.
template <int DT>
__device__ __forceinline__ int count_ge_mem(const void* row, int c0, int c1, float cut, Red& red) {
  const float c = fmaxf(cut, -3.402823466e38f);
  int n = 0;
  for (int e = c0 + (int)threadIdx.x; e < c1; e += kThreads) n += load_logit<DT>(row, e) >= c ? 1 : 0;
  return block_sum_i(n, red);
}

template <int DT>
__device__ __forceinline__ void collect_ge_mem(const void* row, int c0, int c1, float cut, int cap, Smem& sm) {
  const float c = fmaxf(cut, -3.402823466e38f);
  __syncthreads();
  if (threadIdx.x == 0) sm.ch.cnt = 0;
  __syncthreads();
  for (int e = c0 + (int)threadIdx.x; e < c1; e += kThreads) {
    const float x = load_logit<DT>(row, e);
    if (x >= c) {
      const int pos = atomicAdd(&sm.ch.cnt, 1);
      if (pos < cap) sm.ch.cand[pos] = make_float2(x, __int_as_float(e));
    }
  }
  __syncthreads();
}

// Largest window (below mx, in logit units) whose candidate count fits the
// list: bisects between 0 (the maximum alone) and `d` (known to overflow).
template <int DT>
__device__ __forceinline__ float shrink_cut_mem(const void* row, int c0, int c1, float mx, float d, int cap, Red& red) {
  float lo = 0.0f, hi = d, best = kInf;
  if (count_ge_mem<DT>(row, c0, c1, mx, red) <= cap) best = mx;
  for (int it = 0; it < 24 && best != kInf; ++it) {
    const float mid = 0.5f * (lo + hi);
    if (!(mid > lo && mid < hi)) break;
    if (count_ge_mem<DT>(row, c0, c1, mx - mid, red) <= cap) {
      lo = mid;
      best = mx - mid;
    } else {
      hi = mid;
    }
  }
  return best;
}

// One exp per logit: sum of 2^((x - mx) c2) over the thread's logits, and
// (CAND) the candidates of the nucleus window x >= cut.  FMA selects the
// 1-op exponent x*c2 - o (o = mx*c2 rounded), valid when |o| < 2^10.
template <int DT, bool FMA, bool CAND>
__device__ __forceinline__ float exp_pass(uint4 (&buf)[kLoads], float mx, float c2, float o, float cut,
                                          int c0, int cap, Smem& sm) {
  constexpr int VE = Fmt<DT>::VE;
  const int tid = threadIdx.x;
  // An element with x >= cut has a term >= 2^-12 (up to rounding), so a
  // vector whose terms sum below 0.999 * 2^-12 holds no candidate.
  const float hit_sum = 0.999f * 0.000244140625f;
  fence_regs(buf);
  float acc0 = 0.f, acc1 = 0.f, acc2 = 0.f, acc3 = 0.f;
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    float e[VE];
#pragma unroll
    for (int k = 0; k < VE; ++k) {
      const float x = elem<DT>(buf[i], k);
      const float a = FMA ? fmaf(x, c2, -o) : (x - mx) * c2;
      e[k] = __builtin_amdgcn_exp2f(a);
    }
    float s;
    if constexpr (VE == 8)
      s = ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
    else
      s = (e[0] + e[1]) + (e[2] + e[3]);
    if (CAND && s >= hit_sum) append_vec<DT>(buf[i], cut, c0 + (i * kThreads + tid) * VE, cap, sm);
    if ((i & 3) == 0) acc0 += s;
    else if ((i & 3) == 1) acc1 += s;
    else if ((i & 3) == 2) acc2 += s;
    else acc3 += s;
  }
  return (acc0 + acc1) + (acc2 + acc3);
}

// Streaming pass over one chunk held in registers; writes its ChunkRec and
// candidate list.  The kernel instance for MODE handles rows whose
// effective mode is MODE, or plain (top-p >= 1, top-k >= V).
template <int DT, int MODE>
__device__ __forceinline__ void chunk_pass(const KParams& P, const SeqParams& sp, uint4 (&buf)[kLoads],
                                           size_t slot, int c0, int c1, const void* row, Smem& sm) {
  constexpr int VE = Fmt<DT>::VE;
  const int tid = threadIdx.x;
  ChunkRec rec;
  rec.cut = kInf;
  rec.z = 0.0;
  rec.cnt = 0;
  rec.arg = -1;
  rec.flags = 0;
  rec.pad = 0;
  bool has_cands = false;
  bool handled = false;

  if constexpr (MODE == SV_TOPK || MODE == SV_GREEDY) {
    if (sp.mode == MODE) {
      handled = true;
      // maximum and the NaN / +inf check
      fence_regs(buf);
      float mx = -kInf;
      int bad = 0;
#pragma unroll
      for (int i = 0; i < kLoads; ++i)
#pragma unroll
        for (int k = 0; k < VE; ++k) {
          const float x = elem<DT>(buf[i], k);
          mx = fmaxf(mx, x);
          bad |= !(x < kInf);
        }
      if (block_max_i(bad, sm.red)) rec.flags |= kCfNonFinite;
      mx = block_max(mx, sm.red);
      rec.m = mx;
      if constexpr (MODE == SV_GREEDY) {
        fence_regs(buf);
        int best = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < kLoads; ++i)
#pragma unroll
          for (int k = 0; k < VE; ++k)
            if (elem<DT>(buf[i], k) == mx) best = min(best, c0 + (i * kThreads + tid) * VE + k);
        rec.arg = block_min_i(best, sm.red);
      } else {
        has_cands = true;
        const int need = sp.topk;
        float cut = kInf;
        if (need <= P.cap) cut = choose_cut<DT>(buf, mx, 2.0f, need, P.cap, sm.red);
        if (cut != kInf) {
          collect_ge<DT>(buf, cut, c0, P.cap, sm);
          rec.cnt = min(sm.ch.cnt, P.cap);
          rec.cut = sm.ch.cnt <= P.cap ? cut : kInf;
        }
      }
    }
  }
  if constexpr (MODE != SV_GREEDY) {
   if (!handled) {
    // plain and nucleus: one exp per logit
    fence_regs(buf);
    float mx = -kInf;
#pragma unroll
    for (int i = 0; i < kLoads; ++i)
#pragma unroll
      for (int k = 0; k < VE; ++k) mx = fmaxf(mx, elem<DT>(buf[i], k));
    mx = block_max(mx, sm.red);
    rec.m = mx;
    const bool cand = MODE == SV_TOPP && sp.mode == SV_TOPP;
    has_cands = cand;
    if (mx == kInf) {
      rec.flags |= kCfNonFinite;
    } else if (mx == -kInf) {
      // nothing finite in this chunk: only NaN can still make the row invalid
      fence_regs(buf);
      int bad = 0;
#pragma unroll
      for (int i = 0; i < kLoads; ++i)
#pragma unroll
        for (int k = 0; k < VE; ++k) bad |= !(elem<DT>(buf[i], k) < kInf);
      if (block_max_i(bad, sm.red)) rec.flags |= kCfNonFinite;
      rec.cut = -kInf;  // the (empty) candidate list is complete
    } else {
      const float c2 = (float)sp.c2;
      const float o = mx * c2;
      // the fma form is exact up to a common offset |delta| <= 2^-14 when |o| < 2^10
      const bool fma_ok = fabsf(o) < 1024.0f;
      const float cut = mx - kCandLog2 / c2;
      const int cap = P.cap;
      if (cand) {
        __syncthreads();
        if (tid == 0) sm.ch.cnt = 0;
        __syncthreads();
      }
      float zt;
      if (cand) {
        if constexpr (MODE == SV_TOPP) {
          zt = fma_ok ? exp_pass<DT, true, true>(buf, mx, c2, o, cut, c0, cap, sm)
                      : exp_pass<DT, false, true>(buf, mx, c2, o, cut, c0, cap, sm);
        }
      } else {
        zt = fma_ok ? exp_pass<DT, true, false>(buf, mx, c2, o, cut, c0, cap, sm)
                    : exp_pass<DT, false, false>(buf, mx, c2, o, cut, c0, cap, sm);
      }
      const double z = block_sum((double)zt, sm.red);
      // terms were 2^(x*c2 - o); refer them to 2^((x - m) c2) exactly
      const double delta = fma_ok ? (double)mx * (double)c2 - (double)o : 0.0;
      rec.z = z * exp2(-delta);
      if (cand) {
        __syncthreads();
        int n = sm.ch.cnt;
        float used = cut;
        if (n > cap) {
          // too many near the top: narrow the window until the list fits
          used = shrink_cut_mem<DT>(row, c0, c1, mx, kCandLog2 / c2, cap, sm.red);
          if (used != kInf) {
            collect_ge_mem<DT>(row, c0, c1, used, cap, sm);
            n = sm.ch.cnt;
          }
        }
        rec.cnt = min(n, cap);
        rec.cut = (n <= cap) ? used : kInf;
      }
    }
   }
  }

  // publish the chunk's candidates and record
  if (has_cands) {
    float2* dst = P.cands + slot * (size_t)P.cap;
    for (int j = tid; j < rec.cnt; j += kThreads) dst[j] = sm.ch.cand[j];
  }
  if (tid == 0) P.chunks[slot] = rec;
}

// -------------------------------------------------------- selection -----
// MSB-first radix selection over order-preserving keys.  Finds the largest
// logit value T whose inclusive descending cumulative count (top-k) or mass
// (nucleus, fixed point) reaches `target`.  Histograms hold counts and
// fixed-point masses, so the result does not depend on atomic order.
struct SelOut {
  float T;
  bool reached;
  uint32_t n_keep;
  unsigned long long m_keep, m_above;
};

// Source of elements: either the candidate lists of a row's chunks or the
// full row in global memory.
template <int DT>
struct Source {
  const float2* cands;
  int cap;
  int V;
  const ChunkRec* crec;  // in LDS
  size_t slot0;
  int S;
  bool full;
  const void* row;
  float M;
  double c2;
  bool exact_exp;

  template <class F>
  __device__ __forceinline__ void for_each(F&& f) const {
    if (full) {
      for (int e = threadIdx.x; e < V; e += kThreads) f(load_logit<DT>(row, e));
    } else {
      for (int s = 0; s < S; ++s) {
        const float2* c = cands + (slot0 + s) * (size_t)cap;
        const int n = crec[s].cnt;
        for (int j = threadIdx.x; j < n; j += kThreads) f(c[j].x);
      }
    }
  }
  __device__ __forceinline__ unsigned long long mass(float x) const {
    double e;
    if (exact_exp)
      e = exp2(((double)x - (double)M) * c2);
    else
      e = (double)__builtin_amdgcn_exp2f((x - M) * (float)c2);
    return (unsigned long long)(e * kFix + 0.5);
  }
};

template <int DT>
__device__ __forceinline__ SelOut radix_select(const Source<DT>& src, bool by_mass, unsigned long long target, Smem& sm) {
  const int tid = threadIdx.x;
  const int levels = DT == SV_BF16 ? 2 : 4;
  uint32_t pkey = 0, pmask = 0;
  unsigned long long above_c = 0, above_m = 0;
  bool reached = true;
  uint32_t last_c = 0;
  unsigned long long last_m = 0;
  for (int lv = 0; lv < levels; ++lv) {
    const int shift = 24 - 8 * lv;
    __syncthreads();
    sm.mg.hc[tid] = 0;
    sm.mg.hm[tid] = 0;
    __syncthreads();
    src.for_each([&](float x) {
      const uint32_t key = fkey(x);
      if ((key & pmask) == pkey) {
        const uint32_t dg = (key >> shift) & 255u;
        atomicAdd(&sm.mg.hc[dg], 1u);
        atomicAdd(&sm.mg.hm[dg], src.mass(x));
      }
    });
    __syncthreads();
    if (tid < 64) {
      // lane l owns digits 4l..4l+3; suffix sums run from digit 255 down
      const int lane = tid;
      unsigned long long c[4], m[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = sm.mg.hc[4 * lane + j];
        m[j] = sm.mg.hm[4 * lane + j];
      }
      unsigned long long lc = c[0] + c[1] + c[2] + c[3];
      unsigned long long lm = m[0] + m[1] + m[2] + m[3];
      // inclusive suffix over lanes >= lane
      unsigned long long sc = lc, sms = lm;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const unsigned long long yc = __shfl_down(sc, o);
        const unsigned long long ym = __shfl_down(sms, o);
        if (lane + o < 64) {
          sc += yc;
          sms += ym;
        }
      }
      // suffix sums per digit
      unsigned long long suf_c[4], suf_m[4];
      unsigned long long rc = sc - lc, rm = sms - lm;  // digits of higher lanes
#pragma unroll
      for (int j = 3; j >= 0; --j) {
        rc += c[j];
        rm += m[j];
        suf_c[j] = rc;
        suf_m[j] = rm;
      }
      int best = -1;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool ok = by_mass ? (above_m + suf_m[j] >= target) : (above_c + suf_c[j] >= target);
        if (ok) best = 4 * lane + j;
      }
      const int hit = wave_max_i(best);
      int lowest = 256;
#pragma unroll
      for (int j = 3; j >= 0; --j)
        if (c[j] > 0) lowest = 4 * lane + j;
      const int low = wave_min_i(lowest);
      if (lane == 0) {
        sm.mg.sel_hit = hit >= 0 ? 1u : 0u;
        sm.mg.sel_digit = hit >= 0 ? (uint32_t)hit : (low < 256 ? (uint32_t)low : 0u);
      }
    }
    __syncthreads();
    const uint32_t dg = sm.mg.sel_digit;
    if (!sm.mg.sel_hit) reached = false;
    // add everything strictly above the chosen digit
    unsigned long long add_c = 0, add_m = 0;
    if (tid < 64) {
      for (int j = 0; j < 4; ++j) {
        const int d = 4 * tid + j;
        if (d > (int)dg) {
          add_c += sm.mg.hc[d];
          add_m += sm.mg.hm[d];
        }
      }
      for (int o = 32; o > 0; o >>= 1) {
        add_c += __shfl_xor(add_c, o);
        add_m += __shfl_xor(add_m, o);
      }
    }
    __syncthreads();
    if (tid == 0) {
      sm.red.d[0] = __longlong_as_double((long long)add_c);
      sm.red.d[1] = __longlong_as_double((long long)add_m);
      sm.red.d[2] = __longlong_as_double((long long)sm.mg.hc[dg]);
      sm.red.d[3] = __longlong_as_double((long long)sm.mg.hm[dg]);
    }
    __syncthreads();
    above_c += (unsigned long long)__double_as_longlong(sm.red.d[0]);
    above_m += (unsigned long long)__double_as_longlong(sm.red.d[1]);
    last_c = (uint32_t)__double_as_longlong(sm.red.d[2]);
    last_m = (unsigned long long)__double_as_longlong(sm.red.d[3]);
    pkey |= dg << shift;
    pmask |= 255u << shift;
  }
  if (DT == SV_BF16) pkey |= (pkey >> 31) ? 0u : 0xFFFFu;
  SelOut r;
  r.T = key_value(pkey);
  r.reached = reached;
  r.n_keep = (uint32_t)above_c + last_c;
  r.m_keep = above_m + last_m;
  r.m_above = above_m;
  return r;
}

// --------------------------------------------------------- row merge ----
template <int DT>
__device__ __forceinline__ void row_merge(const KParams& P, const SeqParams& sp, int b, size_t rowid, const void* row,
                          int tok, Smem& sm) {
  const int tid = threadIdx.x;
  const int S = P.S;
  const size_t slot0 = rowid * (size_t)S;
  for (int s = tid; s < S; s += kThreads) sm.mg.crec[s] = P.chunks[slot0 + s];
  __syncthreads();
  const int mode = sp.mode;

  float m_s = -kInf;
  int f_s = 0;
  for (int s = tid; s < S; s += kThreads) {
    m_s = fmaxf(m_s, sm.mg.crec[s].m);
    f_s |= (int)sm.mg.crec[s].flags;
  }
  const float M = block_max(m_s, sm.red);
  const int cflags = block_max_i(f_s, sm.red);  // only bit 0 is used

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
      const ChunkRec& c = sm.mg.crec[s];
      if (c.m > -kInf) term += c.z * exp2(((double)c.m - (double)M) * sp.c2);
    }
    Z = block_sum(term, sm.red);
    if (!(Z > 0.0) || !(Z < 1e300)) rr.flags |= SV_ST_NONFINITE;
  }

  if (!(rr.flags & kErrBits)) {
    if (mode == SV_PLAIN) {
      rr.Zs = Z;
    } else if (mode == SV_GREEDY) {
      int best = 0x7fffffff;
      for (int s = tid; s < S; s += kThreads)
        if (sm.mg.crec[s].m == M) best = min(best, sm.mg.crec[s].arg);
      rr.g = block_min_i(best, sm.red);
      rr.T = M;
      rr.n_keep = 1;
    } else {
      float cmax = -kInf;
      for (int s = tid; s < S; s += kThreads) cmax = fmaxf(cmax, sm.mg.crec[s].cut);
      const float C = block_max(cmax, sm.red);
      const bool by_mass = mode == SV_TOPP;
      unsigned long long target;
      if (by_mass) {
        const double t = (double)sp.topp * Z * kFix;
        target = t < 1.0 ? 1ull : (unsigned long long)t;
      } else {
        target = (unsigned long long)sp.topk;
      }
      Source<DT> src{P.cands, P.cap, P.V, sm.mg.crec, slot0, S, false, row, M, sp.c2, true};
      SelOut so;
      bool fast = C < kInf;
      if (fast) {
        so = radix_select<DT>(src, by_mass, target, sm);
        fast = so.reached && so.T >= C;
      }
      if (!fast) {
        src.full = true;
        src.exact_exp = false;
        so = radix_select<DT>(src, by_mass, target, sm);
        rr.flags |= SV_ST_FULLSELECT;
      }
      rr.T = so.T;
      rr.n_keep = (int)so.n_keep;
      rr.Zs = (double)so.m_keep / kFix;
      if (fast && so.n_keep <= (uint32_t)kListMax) rr.flags |= kRfListOk;
      if (by_mass) {
        const double lo = (double)so.m_above / kFix / Z, hi = (double)so.m_keep / kFix / Z;
        if (fabs(lo - (double)sp.topp) < kWindow || fabs(hi - (double)sp.topp) < kWindow)
          rr.flags |= SV_ST_MARGIN;
      }
      if (!(rr.Zs > 0.0)) rr.flags |= SV_ST_EMPTY;
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
  if (tid == 0) P.rows[rowid] = rr;
}

// -------------------------------------------------------- final draw ----
struct Draw {
  int y;
  double S;
  uint32_t flags;
};

// Inverse CDF over the target's kept set (taken from its candidate lists),
// in vocabulary order.  w = (q - p)+ when `resample`, else w = q.
template <int DT>
__device__ __forceinline__ Draw draw_from_list(const KParams& P, const RowRec rq, const bool resample, const RowRec rp,
                               size_t rowq,
                               const void* drow, double u, Smem& sm) {
  const int tid = threadIdx.x;
  const int S = P.S;
  __syncthreads();
  if (tid == 0) sm.fin.n = 0;
  __syncthreads();
  for (int s = 0; s < S; ++s) {
    const ChunkRec cr = P.chunks[rowq * S + s];
    const float2* c = P.cands + (rowq * S + s) * (size_t)P.cap;
    for (int j = tid; j < cr.cnt; j += kThreads) {
      const float2 v = c[j];
      if (v.x >= rq.T) {
        const int pos = atomicAdd(&sm.fin.n, 1);
        if (pos < kListMax) {
          sm.fin.x[pos] = v.x;
          sm.fin.idx[pos] = __float_as_int(v.y);
        }
      }
    }
  }
  __syncthreads();
  const int N = min(sm.fin.n, kListMax);
  // order by vocabulary index (indices are distinct)
  for (int i = tid; i < N; i += kThreads) {
    const int my = sm.fin.idx[i];
    int r = 0;
    for (int j = 0; j < N; ++j) r += sm.fin.idx[j] < my ? 1 : 0;
    sm.fin.sx[r] = sm.fin.x[i];
    sm.fin.sidx[r] = my;
  }
  __syncthreads();
  Draw d;
  d.flags = 0;
  for (int pass = 0; pass < 2; ++pass) {
    const bool resid = resample && pass == 0;
    for (int i = tid; i < N; i += kThreads) {
      const double q = exp2(((double)sm.fin.sx[i] - (double)rq.M) * rq.c2) / rq.Zs;
      double w = q;
      if (resid) {
        const float xp = load_logit<DT>(drow, sm.fin.sidx[i]);
        const double p = xp >= rp.T ? exp2(((double)xp - (double)rp.M) * rp.c2) / rp.Zs : 0.0;
        w = q > p ? q - p : 0.0;
      }
      sm.fin.w[i] = w;
    }
    __syncthreads();
    // prefix in vocabulary order: thread t owns elements 2t, 2t+1
    const int i0 = 2 * tid, i1 = 2 * tid + 1;
    const double w0 = i0 < N ? sm.fin.w[i0] : 0.0, w1 = i1 < N ? sm.fin.w[i1] : 0.0;
    double total;
    const double ex = block_exclusive_scan(w0 + w1, &total, sm.red);
    if (i0 < N) sm.fin.c[i0] = ex + w0;
    if (i1 < N) sm.fin.c[i1] = (ex + w0) + w1;
    __syncthreads();
    d.S = total;
    if (total > 0.0 || pass == 1) break;
    d.flags |= SV_ST_ZERO_RESIDUAL;  // (q - p)+ has no mass: draw from q
    __syncthreads();
  }
  const double target = u * d.S;
  int first = 0x7fffffff, lastnz = -1;
  for (int i = tid; i < N; i += kThreads) {
    if (sm.fin.c[i] > target && sm.fin.w[i] > 0.0) first = min(first, i);
    if (sm.fin.w[i] > 0.0) lastnz = max(lastnz, i);
  }
  first = block_min_i(first, sm.red);
  lastnz = block_max_i(lastnz, sm.red);
  int iy = first <= lastnz ? first : lastnz;
  if (iy < 0) iy = 0;
  d.y = N > 0 ? sm.fin.sidx[iy] : 0;
  if (tid == 0 && N > 0) {
    // margins of interior CDF boundaries
    const double hi = sm.fin.c[iy] / d.S, lo = (sm.fin.c[iy] - sm.fin.w[iy]) / d.S;
    bool nz_before = false, nz_after = false;
    for (int i = 0; i < iy; ++i) nz_before |= sm.fin.w[i] > 0.0;
    for (int i = iy + 1; i < N; ++i) nz_after |= sm.fin.w[i] > 0.0;
    if ((nz_before && u - lo < kWindow) || (nz_after && hi - u < kWindow)) sm.flag = 1;
    else sm.flag = 0;
  }
  __syncthreads();
  if (sm.flag) d.flags |= SV_ST_MARGIN;
  __syncthreads();
  return d;
}

// Inverse CDF over full logit rows re-read from memory, in tiles of
// 256 x 8 tokens (thread t owns tokens 8t..8t+7 of a tile).
template <int DT>
__device__ __forceinline__ double weight(const RowRec& rq, bool use_p, const RowRec& rp, float xq, float xp) {
  double q = 0.0;
  if (xq >= rq.T) q = (double)__builtin_amdgcn_exp2f((xq - rq.M) * (float)rq.c2) / rq.Zs;
  if (!use_p) return q;
  double p = 0.0;
  if (xp >= rp.T) p = (double)__builtin_amdgcn_exp2f((xp - rp.M) * (float)rp.c2) / rp.Zs;
  return q > p ? q - p : 0.0;
}

template <int DT>
__device__ __forceinline__ Draw draw_from_rows(const KParams& P, const RowRec rq, const bool resample, const RowRec rp,
                               const void* qrow,
                               const void* prow, double u, Smem& sm) {
  const int tid = threadIdx.x;
  const int V = P.V;
  constexpr int TILE = kThreads * 8;
  Draw d;
  d.flags = SV_ST_REREAD;
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
      lo = S - 0.0;
      hi = S;
    }
    d.y = y;
    if (nz_lo < y && u - lo / S < kWindow) d.flags |= SV_ST_MARGIN;
    if (nz_hi > y && hi / S - u < kWindow) d.flags |= SV_ST_MARGIN;
    break;
  }
  return d;
}

template <int DT>
__device__ __forceinline__ const void* row_ptr(const KParams& P, int b, bool tgt, int t) {
  constexpr int ES = Fmt<DT>::ES;
  const size_t r = tgt ? ((size_t)b * (P.K_max + 1) + t) : ((size_t)b * P.K_max + t);
  return static_cast<const char*>(tgt ? P.target : P.draft) + r * (size_t)P.V * ES;
}

template <int DT>
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
__device__ __forceinline__ void finalize(const KParams& P, const SeqParams& sp, int b, Smem& sm) {
  const int tid = threadIdx.x;
  const int Kb = sp.Kb, KM = P.K_max, R = P.R;
  const uint64_t g = P.row_offset + (uint64_t)b;
  const size_t rbase = (size_t)b * R;
  // OR of the row records' flags
  uint32_t st;
  {
    uint32_t v = 0;
    for (int t = tid; t <= Kb; t += kThreads) v |= P.rows[rbase + t].flags;
    for (int t = tid; t < Kb; t += kThreads) v |= P.rows[rbase + KM + 1 + t].flags;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v |= (uint32_t)__shfl_xor((int)v, o);
    __syncthreads();
    if ((tid & 63) == 0) sm.red.i[tid >> 6] = (int)v;
    __syncthreads();
    st = (uint32_t)(sm.red.i[0] | sm.red.i[1] | sm.red.i[2] | sm.red.i[3]);
    __syncthreads();
  }
  st &= ~kRfListOk;
  if (st & kErrBits) {
    write_error<DT>(P, b, st & kErrBits);
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
    sm.red.i[0] = n;
    sm.red.i[1] = (int)s2;
  }
  __syncthreads();
  const int n = sm.red.i[0];
  st |= (uint32_t)sm.red.i[1];
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
    d = draw_from_list<DT>(P, rq, resample, rp, rbase + n,
                           resample ? row_ptr<DT>(P, b, false, n) : nullptr, u, sm);
  } else {
    d = draw_from_rows<DT>(P, rq, resample, rp, row_ptr<DT>(P, b, true, n),
                           resample ? row_ptr<DT>(P, b, false, n) : nullptr, u, sm);
  }
  st |= d.flags;
  for (int i = tid; i <= KM; i += kThreads) {
    int v = -1;
    if (i < n) v = P.tokens[(size_t)b * KM + i];
    else if (i == n) v = d.y;
    P.out_tokens[(size_t)b * (KM + 1) + i] = v;
  }
  if (tid == 0) {
    P.accepted[b] = n;
    if (P.status) P.status[b] = st & ~kRfListOk;
  }
}

// ------------------------------------------------------------ kernel ----
template <int DT, bool VEC, int MODE>
__global__ __launch_bounds__(kThreads) void verify_kernel(const KParams P) {
  __shared__ Smem sm;
  const int tid = threadIdx.x;
  const int S = P.S, R = P.R;
  const size_t blk = blockIdx.x;
  const int b = P.b_base + (int)(blk / ((size_t)R * S));
  const int rem = (int)(blk % ((size_t)R * S));
  const int r = rem / S, c = rem % S;

  // Each sequence is handled by the instance of its sampling mode (an invalid
  // mode value by the plain instance, which reports the error).
  const int raw_mode = P.mode ? (int)P.mode[b] : P.dmode;
  if ((raw_mode >= SV_PLAIN && raw_mode <= SV_GREEDY ? raw_mode : SV_PLAIN) != MODE) return;
  const SeqParams sp = load_params(P, b);
  if (!sp.valid) {
    if (r == 0 && c == 0) write_error<DT>(P, b, SV_ST_PARAM);
    return;
  }
  const bool tgt = r <= P.K_max;
  const int t = tgt ? r : r - P.K_max - 1;
  if (tgt ? (t > sp.Kb) : (t >= sp.Kb)) return;  // padding row: never read

  const void* row = row_ptr<DT>(P, b, tgt, t);
  const size_t rowid = (size_t)b * R + r;
  const size_t slot = rowid * S + c;
  const int c0 = c * P.L;
  const int c1 = min(P.V, c0 + P.L);

  {
    uint4 buf[kLoads];
    load_chunk<DT, VEC>(buf, static_cast<const char*>(row), c0, c1);
    chunk_pass<DT, MODE>(P, sp, buf, slot, c0, c1, row, sm);
  }

  // last chunk of the row merges it
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const uint32_t old = atomicAdd(&P.rowctr[rowid], 1u);
    sm.flag = old == (uint32_t)(S - 1);
    if (sm.flag) {
      atomicExch(&P.rowctr[rowid], 0u);
      __threadfence();
    }
  }
  __syncthreads();
  if (!sm.flag) return;

  const int tok = (t < sp.Kb) ? P.tokens[(size_t)b * P.K_max + t] : INT32_MIN;
  row_merge<DT>(P, sp, b, rowid, row, tok, sm);

  // last row of the sequence finalizes it
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const uint32_t old = atomicAdd(&P.seqctr[b], 1u);
    sm.flag = old == (uint32_t)(2 * sp.Kb);
    if (sm.flag) {
      atomicExch(&P.seqctr[b], 0u);
      __threadfence();
    }
  }
  __syncthreads();
  if (!sm.flag) return;
  finalize<DT>(P, sp, b, sm);
}

}  // namespace

template <int DT, bool VEC>
static void launch_mode(const KParams& p, int mode, dim3 grid, hipStream_t stream) {
  const dim3 block(kThreads);
  switch (mode) {
    case SV_PLAIN: hipLaunchKernelGGL((verify_kernel<DT, VEC, SV_PLAIN>), grid, block, 0, stream, p); break;
    case SV_TOPK: hipLaunchKernelGGL((verify_kernel<DT, VEC, SV_TOPK>), grid, block, 0, stream, p); break;
    case SV_TOPP: hipLaunchKernelGGL((verify_kernel<DT, VEC, SV_TOPP>), grid, block, 0, stream, p); break;
    default: hipLaunchKernelGGL((verify_kernel<DT, VEC, SV_GREEDY>), grid, block, 0, stream, p); break;
  }
}

hipError_t launch_verify(const KParams& p, int dtype, bool vec, int nseq, hipStream_t stream) {
  const size_t blocks = (size_t)nseq * p.R * p.S;
  if (blocks == 0) return hipSuccess;
  const dim3 grid((unsigned)blocks);
  // One instance per sampling mode present: with a per-row mode array every
  // instance runs (each skips the sequences of other modes).
  for (int mode = SV_PLAIN; mode <= SV_GREEDY; ++mode) {
    if (!p.mode && mode != p.dmode) continue;
    if (dtype == SV_BF16) {
      if (vec) launch_mode<SV_BF16, true>(p, mode, grid, stream);
      else launch_mode<SV_BF16, false>(p, mode, grid, stream);
    } else {
      if (vec) launch_mode<SV_F32, true>(p, mode, grid, stream);
      else launch_mode<SV_F32, false>(p, mode, grid, stream);
    }
  }
  return hipGetLastError();
}

}  // namespace sv
