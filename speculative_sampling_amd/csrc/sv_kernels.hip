// gfx950 kernels of the verify-and-resample step of speculative sampling.
//
// A call runs two stages on the caller's stream; the kernel boundary orders
// them, so no work-group ever waits for another:
//
//   chunk_kernel    one wave per chunk of a logit row.  Every used row
//                   (target positions 0..K_b, draft positions 0..K_b-1) is
//                   split into chunks of 8192 bf16 / 4096 fp32 logits; each
//                   wave streams its chunk from HBM into registers exactly
//                   once and reduces it: the sum of the terms 2^((x - m) c2)
//                   and the maximum, the candidate vectors of the nucleus /
//                   top-k threshold search, the greedy argmax.  One instance
//                   per sampling mode keeps each mode's registers minimal.
//   seq_kernel      one work-group per sequence.  Each wave merges one row:
//                   log-sum-exp over the chunks, radix selection of the
//                   threshold over the candidates cached in LDS, kept mass,
//                   the probability of the row's draft token and, for target
//                   rows, the kept set in vocabulary order.  Then the accept
//                   walk, the first rejection, the resample from
//                   normalize((q - p)+) or the bonus draw, and the outputs.
//
// The step follows the pages' rule (FDE Interviews breakdown of Chen et al.,
// section 01 and its figure; paperlayer.ai summary of arXiv 2302.01318,
// "Modified Rejection Sampling"): keep d_t with probability
// min(1, q_t(d_t) / p_t(d_t)), resample the first rejection from the
// normalised positive part of q - p, else draw a bonus token from the
// target's last position; sampling controls are applied to both models
// before the rejection step.  The pages describe no GPU kernel; everything
// below is this library's own design for gfx950.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sv_internal.h"

namespace sv {
namespace {

constexpr float kInf = __builtin_inff();

// Streaming 16-byte load: every logit is read once by the streaming pass, so
// its loads carry the non-temporal hint (measured on MI355X: the read rate
// of the pass rises from 5.65 to 6.03 TB/s with it).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
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

// 2^a for |a| < 2^-14, the size of the rounding error of an fp32 product
// such as M * c2 against its fp64 value: a Taylor polynomial in t = a ln 2,
// whose omitted terms are below 1e-19 relative.  Larger arguments go to
// the fp64 exp2.
__device__ __forceinline__ double exp2_small(double a) {
  if (fabs(a) < 6.103515625e-05) {
    const double t = a * 0.69314718055994530942;
    return 1.0 + t * (1.0 + t * (0.5 + t * (1.0 / 6.0)));
  }
  return exp2(a);
}

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
// Wave scans and reductions by DPP lane moves: shifts of 1, 2, 4 and 8
// lanes within each row of 16, then the last lane of row 0 / rows 0-1
// broadcast into the rows above; lanes with no source take the identity.
// Callers run them with the whole wave active.  Reductions read the result
// from lane 63, so every lane gets the same bits.
template <int CTRL, int ROWS, class T>
__device__ __forceinline__ T dpp_move(T v, T id) {
  static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32- or 64-bit values");
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(T, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, id), __builtin_bit_cast(int, v),
                                                             CTRL, ROWS, 0xf, false));
  } else {
    const unsigned long long a = __builtin_bit_cast(unsigned long long, v);
    const unsigned long long b = __builtin_bit_cast(unsigned long long, id);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)b, (int)(uint32_t)a, CTRL, ROWS, 0xf, false);
    const uint32_t hi =
        (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)(b >> 32), (int)(uint32_t)(a >> 32), CTRL, ROWS, 0xf, false);
    return __builtin_bit_cast(T, ((unsigned long long)hi << 32) | lo);
  }
}
template <class T, class Op>
__device__ __forceinline__ T wave_scan(T v, T id, Op op) {
  v = op(v, dpp_move<0x111, 0xf>(v, id));  // row_shr:1
  v = op(v, dpp_move<0x112, 0xf>(v, id));  // row_shr:2
  v = op(v, dpp_move<0x114, 0xf>(v, id));  // row_shr:4
  v = op(v, dpp_move<0x118, 0xf>(v, id));  // row_shr:8
  v = op(v, dpp_move<0x142, 0xa>(v, id));  // row_bcast:15
  v = op(v, dpp_move<0x143, 0xc>(v, id));  // row_bcast:31
  return v;
}
// The value of lane L (wave-uniform) for every lane.
template <class T>
__device__ __forceinline__ T lane_at(T v, int L) {
  static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32- or 64-bit values");
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), L));
  } else {
    const unsigned long long a = __builtin_bit_cast(unsigned long long, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)a, L);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(a >> 32), L);
    return __builtin_bit_cast(T, ((unsigned long long)hi << 32) | lo);
  }
}
template <class T>
__device__ __forceinline__ T lane63(T v) {
  return lane_at(v, kWave - 1);
}
__device__ __forceinline__ float wave_max(float v) {
  return lane63(wave_scan(v, -kInf, [](float a, float b) { return fmaxf(a, b); }));
}
__device__ __forceinline__ double wave_sum(double v) {
  return lane63(wave_scan(v, 0.0, [](double a, double b) { return a + b; }));
}
__device__ __forceinline__ int wave_min_i(int v) {
  return lane63(wave_scan(v, 0x7fffffff, [](int a, int b) { return min(a, b); }));
}
__device__ __forceinline__ int wave_max_i(int v) {
  return lane63(wave_scan(v, (int)0x80000000, [](int a, int b) { return max(a, b); }));
}
__device__ __forceinline__ uint32_t wave_or_u(uint32_t v) {
  return lane63(wave_scan(v, 0u, [](uint32_t a, uint32_t b) { return a | b; }));
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
      for (int i = 0; i < kLoads; ++i) buf[i] = load_stream(&base[i * kWave + lane]);
    } else {
      // the row's last chunk: clamped addresses, -inf past c1
      const int nvec = (c1 - c0) / VE;
#pragma unroll
      for (int i = 0; i < kLoads; ++i) buf[i] = load_stream(&base[min(i * kWave + lane, nvec - 1)]);
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

// The largest logit of each of the lane's vectors (vmax[i]) and the chunk
// maximum, with whether the chunk holds a NaN or +inf, in one pass.
template <int DT>
__device__ __forceinline__ float vector_maxima(const uint4 (&buf)[kLoads], float (&vmax)[kLoads], bool* bad) {
  constexpr int VE = Fmt<DT>::VE;
  float mx = -kInf;
  int nf = 0;
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    float m = -kInf;
#pragma unroll
    for (int k = 0; k < VE; ++k) {
      const float x = elem<DT>(buf[i], k);
      m = fmaxf(m, x);
      nf |= !(x < kInf);
    }
    vmax[i] = m;
    mx = fmaxf(mx, m);
  }
  *bad = __ballot(nf) != 0;
  return wave_max(mx);
}

// Number of the chunk's vectors whose largest logit is >= cut (wave
// ballots over the 16 maxima of each lane).
__device__ __forceinline__ int count_vectors_ge(const float (&vmax)[kLoads], float cut) {
  const float c = fmaxf(cut, -kMaxFinite);  // -inf logits are never candidates
  int n = 0;
#pragma unroll
  for (int i = 0; i < kLoads; ++i) n += __popcll(__ballot(vmax[i] >= c));
  return n;
}

// Top-k window: a cut such that the number of vectors holding a logit >= cut
// lies in [need, cap].  The list holds those vectors (at most cap), and they
// hold at least need logits >= cut.  Grows the window below the chunk max
// from d (logit units) until `need` vectors are in, then bisects while the
// list would overflow.  +inf when none exists.
__device__ __forceinline__ float choose_cut(const float (&vmax)[kLoads], float mx, float d, int need, int cap) {
  float lo = 0.0f;  // window known to hold < need vectors (or 0)
  float cut = mx - d;
  int n = count_vectors_ge(vmax, cut);
  for (int it = 0; n < need && it < 64; ++it) {
    lo = d;
    d *= 4.0f;
    cut = mx - d;
    if (!(cut > -kMaxFinite)) {  // the window covers every finite logit
      cut = -kInf;
      n = count_vectors_ge(vmax, cut);
      break;
    }
    n = count_vectors_ge(vmax, cut);
  }
  if (n <= cap) return cut;
  float hi = d;
  for (int it = 0; it < 40; ++it) {
    const float mid = 0.5f * (lo + hi);
    if (!(mid > lo && mid < hi)) break;
    const float cm = mx - mid;
    const int nm = count_vectors_ge(vmax, cm);
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

// Lists each vector flagged in `mask` as (index of its first logit, key),
// in (vector, lane) order, i.e. increasing vocabulary index; returns how
// many there are (entries beyond cap are dropped).  key[i] is the vector's
// largest term 2^(x c2 - o) (nucleus) or its largest logit (top-k).
__device__ __forceinline__ int list_vectors(int2* de, uint32_t mask, const float* key, int c0, int ve, int cap,
                                            int lane) {
  const uint64_t below = (1ull << lane) - 1ull;
  const int e0 = c0 + lane * ve;  // first index of the lane's vector in slot 0
  int n = 0;
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const bool h = (mask >> i) & 1u;
    const uint64_t bal = __ballot(h);
    if (bal) {  // slots with no listed vector cost one ballot
      if (h) {
        const int pos = n + __popcll(bal & below);
        if (pos < cap) de[pos] = make_int2(e0 + i * kWave * ve, __float_as_int(key[i]));
      }
      n += __popcll(bal);
    }
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
  ps.ma = ps.st == 0 ? ((double)log2f(em) + (double)o) * (1.0 / (double)c2) : -1e300;
}

// Finishes a plain / nucleus chunk.  A nucleus chunk lists every logit
// x >= g - 10/c2, where g >= the chunk maximum is the largest maximum among
// the chunks of the same row in this work-group (lists that overflow are
// retried with 8 and 6); its vectors are flagged from their largest terms
// with a 2^-8 margin in the exponent, a superset of those holding one.
template <int DT>
__device__ __forceinline__ void plain_finish(const KParams& P, const PlainStats& ps, float c2, bool cand,
                                             double g, size_t slot, int c0, int lane, ChunkRec& rec) {
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
  rec.o = ps.o;
  // refer the sum to m: 2^(x c2 - o) = 2^((x - m) c2) 2^(m c2 - o)
  // (the exponent is -log2 of the largest term, within [-2^7, 0]: fp32
  // exp2 keeps the ~1e-7 relative error of the terms themselves)
  rec.z = ps.zw * (double)exp2f((float)((double)ps.o - (double)m * (double)c2));
  if (cand) {
    int2* de = P.cent + slot * (size_t)P.cap;
    int n = 0;
    float cut = kInf;
    const double ic2 = 1.0 / (double)c2;
    for (int attempt = 0; attempt < 3; ++attempt) {
      cut = (float)(g - (attempt == 0 ? kCandLog2 : attempt == 1 ? 8.0 : 6.0) * ic2);
      // x >= cut implies a term >= 2^(cut c2 - o) up to roundings far below the margin
      const float thr = exp2f((float)((double)cut * (double)c2 - (double)ps.o) - 0.00390625f);
      uint32_t mask = 0;
#pragma unroll
      for (int i = 0; i < kLoads; ++i) mask |= ps.emax[i] >= thr ? (1u << i) : 0u;
      n = list_vectors(de, mask, ps.emax, c0, Fmt<DT>::VE, P.cap, lane);
      if (n <= P.cap) break;
    }
    rec.cnt = n <= P.cap ? n : 0;
    rec.cut = n <= P.cap ? cut : kInf;  // +inf: incomplete, the merge falls back to the full row
  }
}

// Template mode of the streaming instance for calls with a per-sequence
// mode array: every wave takes its own row's path, in one launch.
constexpr int kAnyMode = 4;

// Streaming pass: one wave per chunk.  The instance for MODE handles the
// sequences whose sampling mode is MODE; those whose effective mode is plain
// (top-p >= 1, top-k >= V) take the plain path.
// Work-groups are handed to the 8 XCDs in turn (work-group j to XCD
// j mod 8), and the sequence kernel's work-group b runs on XCD b mod 8.
// When every sequence spans a whole number Q of streaming work-groups and
// the launch holds a multiple of 8 sequences, hardware work-group j takes
// the logical work-group that keeps all of sequence b's chunks on XCD
// b mod 8 as well (a permutation of [0, 8 Q n)); otherwise the identity.
__device__ __forceinline__ uint32_t xcd_logical_wg(uint32_t j, int nseq, int rs) {
  constexpr uint32_t kXcd = 8;
  constexpr int wpg = kThreads / kWave;  // waves (chunks) per streaming work-group
  if (rs % wpg != 0 || nseq % (int)kXcd != 0) return j;
  const uint32_t Q = (uint32_t)(rs / wpg);
  const uint32_t x = j % kXcd, k = j / kXcd;
  return (x + kXcd * (k / Q)) * Q + k % Q;
}

template <int DT, bool VEC, int MODE>
__global__ __launch_bounds__(kThreads, (MODE == SV_TOPK || MODE == kAnyMode) ? 3 : 1) void chunk_kernel(
    const KParams P) {
  constexpr int VE = Fmt<DT>::VE;
  constexpr int kWaves = kThreads / kWave;
  // which paths this instance holds
  constexpr bool kAny = MODE == kAnyMode;
  constexpr bool kTopk = MODE == SV_TOPK || kAny;
  constexpr bool kGreedy = MODE == SV_GREEDY || kAny;
  constexpr bool kTopp = MODE == SV_TOPP || kAny;
  constexpr bool kPlain = MODE != SV_GREEDY;
  // [0]: the top-k cut exchange, [1]: the nucleus window exchange
  __shared__ float s_max[2][kWaves];
  __shared__ int s_key[2][kWaves];
  const int lane = (int)__lane_id();
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  const int S = P.S, R = P.R;
  const uint32_t gw = xcd_logical_wg(blockIdx.x, P.b_end - P.b_base, R * S) * (uint32_t)kWaves + (uint32_t)wv;
  const int b = P.b_base + (int)(gw / (uint32_t)(R * S));
  const int rem = (int)(gw % (uint32_t)(R * S));
  const int r = rem / S, c = rem % S;
  // no early return: the work-group meets at its barriers
  bool active = b < P.b_end && (kAny || raw_mode(P, b) == MODE);
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
  rec.o = 0.0f;
  uint4 buf[kLoads];
  if (active) load_chunk<DT, VEC>(buf, row, c0, c1, lane);

  const bool is_topk = kTopk && active && sp.mode == SV_TOPK;  // wave-uniform
  const bool special = is_topk || (kGreedy && active && sp.mode == SV_GREEDY);
  float kcut = kInf;    // top-k: this chunk's own cut (+inf: none)
  float vmax[kLoads];   // top-k: each vector's largest logit
  if (special) {
    bool bad;
    const float mx = is_topk ? vector_maxima<DT>(buf, vmax, &bad) : chunk_max<DT>(buf, &bad);
    rec.m = mx;
    if (bad) {
      rec.flags |= kCfNonFinite;
    } else if (!is_topk) {  // greedy
      int best = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < kLoads; ++i)
#pragma unroll
        for (int k = 0; k < VE; ++k)
          if (elem<DT>(buf[i], k) == mx) best = min(best, c0 + (i * kWave + lane) * VE + k);
      rec.arg = wave_min_i(best);
    } else {
      const int need = sp.topk, cap = P.cap;
      // at most about 2k candidate vectors per chunk keep the row's list short
      if (need <= cap) kcut = choose_cut(vmax, mx, 2.0f, need, min(cap, max(2 * need, 64)));
    }
  }
  if constexpr (kTopk) {
    // Each chunk lists against the largest cut among this work-group's
    // chunks of the same row: the chunk that set it holds >= k vectors at
    // or above it, every chunk's list stays complete above it, and no list
    // grows (the shared cut is at least the chunk's own).
    const bool hascut = is_topk && kcut != kInf;
    if (lane == 0) {
      s_key[0][wv] = hascut ? (int)(gw / (uint32_t)S) : -1;
      s_max[0][wv] = hascut ? kcut : -kInf;
    }
    __syncthreads();
    if (hascut) {
      const int key = (int)(gw / (uint32_t)S);
      float cut = kcut;
#pragma unroll
      for (int w = 0; w < kWaves; ++w)
        if (s_key[0][w] == key) cut = fmaxf(cut, s_max[0][w]);
      const int cap = P.cap;
      const float c = fmaxf(cut, -kMaxFinite);
      uint32_t mask = 0;
#pragma unroll
      for (int i = 0; i < kLoads; ++i) mask |= vmax[i] >= c ? (1u << i) : 0u;
      const int n = list_vectors(P.cent + slot * (size_t)cap, mask, vmax, c0, VE, cap, lane);
      rec.cnt = min(n, cap);
      rec.cut = n <= cap ? cut : kInf;
    }
  }
  if constexpr (kPlain) {
    const bool plain = active && !special;
    const bool cand = plain && kTopp && sp.mode == SV_TOPP;
    PlainStats ps;
    ps.st = 1;
    ps.ma = -1e300;
    if (plain) plain_stats<DT, VEC>(buf, c2, row, c0, c1, lane, ps);
    double g = ps.ma;
    if constexpr (kTopp) {
      // the largest chunk maximum among this work-group's chunks of the same row
      if (lane == 0) {
        s_key[1][wv] = cand ? (int)(gw / (uint32_t)S) : -1;
        s_max[1][wv] = ps.st == 0 ? (float)ps.ma : -kInf;
      }
      __syncthreads();
      const int key = cand ? (int)(gw / (uint32_t)S) : -2;
#pragma unroll
      for (int w = 0; w < kWaves; ++w)
        if (s_key[1][w] == key) g = fmax(g, (double)s_max[1][w]);
    }
    if (plain) plain_finish<DT>(P, ps, c2, cand, g, slot, c0, lane, rec);
  }
  if (active && lane == 0) P.chunks[slot] = rec;
}

// ===================================================== sequence kernel ====
//
// One work-group per sequence.  Wave w merges rows w, w + kSeqWaves, ... of
// the sequence with wave-level operations only: log-sum-exp over the chunk
// records, the top-k / nucleus threshold by radix selection over the
// candidates cached in LDS, the probability of the row's draft token and,
// for target rows, the kept set in vocabulary order.  After one barrier the
// work-group runs the accept walk, finds the first rejection and draws the
// resampled or bonus token.

constexpr int kSeqThreads = kSeqWaves * kWave;
constexpr int kRowCache = 768;   // candidate logits of one row held in LDS
constexpr int kDrawTiles = 8;   // tiles of a row draw whose loads are in flight together
constexpr int kVecList = 768;   // candidate vectors of one row that pass the row's cut
constexpr int kMaxRows = 2 * kMaxK + 1;

// Orders the wave's LDS accesses (and keeps the compiler from moving them).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ unsigned long long wave_incl_scan_u64(unsigned long long v, int) {
  return wave_scan(v, 0ull, [](unsigned long long a, unsigned long long b) { return a + b; });
}
__device__ __forceinline__ double wave_incl_scan(double v, int) {
  return wave_scan(v, 0.0, [](double a, double b) { return a + b; });
}
__device__ __forceinline__ int wave_incl_scan_i(int v, int) {
  return wave_scan(v, 0, [](int a, int b) { return a + b; });
}

struct WaveSmem {
  float cx[kRowCache];  // cached candidates: logit and vocabulary index;
  int ci[kRowCache];    //   afterwards the kept set in vocabulary order
  int vi[kVecList];     // first index of each candidate vector; afterwards
                        //   the draft's logits at the kept set (float bits)
  uint32_t hc[256];     // radix histogram: counts and fixed-point masses
  unsigned long long hm[256];
  int pre[kWave];       // list start of each chunk of the current batch
  float thr[kWave];     // key threshold of each chunk of the current batch
};

struct SmemSeq {
  WaveSmem w[kSeqWaves];
  RowRec rows[kMaxRows];
  double rd[kSeqWaves];
  int ri[kSeqWaves];
  uint32_t misc[4];
  double rx[2];
  double ua[kWave];  // uniforms of the accept tests at positions 0..63, and of
  double ud[kWave];  //   the resample (t < K_b) or bonus (t = K_b) draws
};

struct SelOut {
  float T;
  bool reached;
  uint32_t n_keep;
  unsigned long long m_keep, m_above;
};

// One digit of a selection: scans the 256-bin histogram in ws from the top
// digit down, with the counts and masses above it (above_c, above_m), for
// the first digit whose inclusive cumulative count (top-k) or fixed-point
// mass (nucleus) reaches `target`; without one (not reached), the lowest
// non-empty digit.  Adds the exclusive sums at the digit to above_*, and
// returns the digit with its own count and mass in last_*.
__device__ __forceinline__ int pick_digit(const WaveSmem& ws, bool by_mass, unsigned long long target,
                                          unsigned long long& above_c, unsigned long long& above_m,
                                          unsigned long long& last_c, unsigned long long& last_m, bool& reached,
                                          int lane) {
  // lane l holds digits 255 - 4l - j, j = 0..3: descending over the wave
  unsigned long long c[4], m[4], lc = 0, lm = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    c[j] = ws.hc[255 - 4 * lane - j];
    m[j] = ws.hm[255 - 4 * lane - j];
    lc += c[j];
    lm += m[j];
  }
  const unsigned long long ec = wave_incl_scan_u64(lc, lane) - lc, em = wave_incl_scan_u64(lm, lane) - lm;
  int bj = -1, nj = -1;
  unsigned long long xc = 0, xm = 0, yc = 0, ym = 0;  // exclusive sums at the hit / last non-empty digit
  unsigned long long rc = ec, rm = em;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bool ok = by_mass ? (above_m + rm + m[j] >= target) : (above_c + rc + c[j] >= target);
    if (ok && bj < 0) {
      bj = j;
      xc = rc;
      xm = rm;
    }
    if (c[j] > 0) {
      nj = j;
      yc = rc;
      ym = rm;
    }
    rc += c[j];
    rm += m[j];
  }
  const uint64_t hit = __ballot(bj >= 0);
  int L, J;
  unsigned long long ac, am;
  if (hit) {
    L = __ffsll((long long)hit) - 1;
    J = lane_at(bj, L);
    ac = lane_at(xc, L);
    am = lane_at(xm, L);
  } else {
    reached = false;  // keep everything: the lowest non-empty digit
    const uint64_t ne = __ballot(nj >= 0);
    L = ne ? 63 - __clzll((long long)ne) : kWave - 1;
    J = ne ? lane_at(nj, L) : 3;
    ac = lane_at(yc, L);
    am = lane_at(ym, L);
  }
  const int dg = 255 - 4 * L - J;
  above_c += ac;
  above_m += am;
  last_c = ws.hc[dg];
  last_m = ws.hm[dg];
  return dg;
}

__device__ __forceinline__ void clear_histogram(WaveSmem& ws, int lane) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    ws.hc[lane + kWave * j] = 0;
    ws.hm[lane + kWave * j] = 0;
  }
  wave_sync();
}

// MSB-first radix selection (8-bit digits) over order-preserving keys: the
// largest logit value T whose inclusive descending cumulative count (top-k)
// or fixed-point mass (nucleus) reaches `target`.  Integer histograms make
// the result independent of the order of the atomic additions.  each(f)
// calls f(x, mass) for this lane's share of the elements.
template <int DT, class Each>
__device__ __forceinline__ SelOut wave_select(Each&& each, bool by_mass, unsigned long long target, WaveSmem& ws,
                                              int lane) {
  const int levels = DT == SV_BF16 ? 2 : 4;
  uint32_t pkey = 0, pmask = 0;
  unsigned long long above_c = 0, above_m = 0, last_c = 0, last_m = 0;
  bool reached = true;
  for (int lv = 0; lv < levels; ++lv) {
    const int shift = 24 - 8 * lv;
    clear_histogram(ws, lane);
    each([&](float x, unsigned long long m) {
      const uint32_t key = fkey(x);
      if ((key & pmask) == pkey) {
        const uint32_t dg = (key >> shift) & 255u;
        atomicAdd(&ws.hc[dg], 1u);
        atomicAdd(&ws.hm[dg], m);
      }
    });
    wave_sync();
    const int dg = pick_digit(ws, by_mass, target, above_c, above_m, last_c, last_m, reached, lane);
    pkey |= (uint32_t)dg << shift;
    pmask |= 255u << shift;
    wave_sync();
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

// Whether bf16 elements known to lie in [lo, hi] span fewer than 256
// 16-bit keys: then one histogram level over the keys themselves gives the
// selection (select_narrow).
__device__ __forceinline__ bool narrow_range(float lo, float hi) {
  return lo <= hi && (fkey(hi) >> 16) - (fkey(lo) >> 16) < 256u;
}

// The same selection as wave_select in one level, for bf16 elements in
// [lo, hi] with narrow_range(lo, hi): digit 255 - (key(hi) - key).
template <class Each>
__device__ __forceinline__ SelOut select_narrow(Each&& each, bool by_mass, unsigned long long target, WaveSmem& ws,
                                                int lane, float hi) {
  const uint32_t kb = (fkey(hi) >> 16) - 255u;  // the key of digit 0
  unsigned long long above_c = 0, above_m = 0, last_c = 0, last_m = 0;
  bool reached = true;
  clear_histogram(ws, lane);
  each([&](float x, unsigned long long m) {
    const uint32_t dg = min(255u, (fkey(x) >> 16) - kb);  // the bound only guards the index
    atomicAdd(&ws.hc[dg], 1u);
    atomicAdd(&ws.hm[dg], m);
  });
  wave_sync();
  const int dg = pick_digit(ws, by_mass, target, above_c, above_m, last_c, last_m, reached, lane);
  wave_sync();
  uint32_t pkey = (kb + (uint32_t)dg) << 16;
  pkey |= (pkey >> 31) ? 0u : 0xFFFFu;
  SelOut r;
  r.T = key_value(pkey);
  r.reached = reached;
  r.n_keep = (uint32_t)(above_c + last_c);
  r.m_keep = above_m + last_m;
  r.m_above = above_m;
  return r;
}

// Selection over elements known to lie in [lo, hi].
template <int DT, class Each>
__device__ __forceinline__ SelOut select_bounded(Each&& each, bool by_mass, unsigned long long target,
                                                 WaveSmem& ws, int lane, float lo, float hi) {
  if constexpr (DT == SV_BF16) {
    if (narrow_range(lo, hi)) return select_narrow(each, by_mass, target, ws, lane, hi);
  }
  return wave_select<DT>(each, by_mass, target, ws, lane);
}

// Fixed-point mass of a logit, in units of the row's largest term:
// 2^((x - M) c2) = 2^(x c2 - oM) 2^(oM - M c2), with oM = M c2 in fp32 and
// the second factor (fM) exact in fp64.
__device__ __forceinline__ unsigned long long mass_of(float x, float c2, float oM, double fM) {
  return (unsigned long long)((double)__builtin_amdgcn_exp2f(fmaf(x, c2, -oM)) * fM * kFix + 0.5);
}

// Collects, in list order (chunk, vector, lane: increasing vocabulary
// index), the first index of every listed candidate vector of the row whose
// key reaches the threshold of its chunk for the cut Cu, into ws.vi;
// returns how many there are (entries beyond kVecList are counted only).
// keep_keys also stores each kept entry's key in ws.cx.  The key of a
// nucleus vector is its largest term 2^(x c2 - o_chunk) (the
// threshold 2^(Cu c2 - o_chunk - 2^-8) keeps every vector holding x >= Cu);
// that of a top-k vector its largest logit (threshold Cu).
template <class RecAt>
__device__ __forceinline__ int filter_listed(const KParams& P, size_t slot0, RecAt&& rec_at, float Cu, float c2,
                                             bool terms, int lane, WaveSmem& ws, bool keep_keys = false) {
  constexpr int kBatch = 16;
  const int S = P.S;
  const uint64_t below = (1ull << lane) - 1ull;
  int nv = 0;
  for (int s0 = 0; s0 < S; s0 += kWave) {
    const int s = s0 + lane;
    int cnt = 0;
    float th = -kInf;
    if (s < S) {
      const ChunkRec c = rec_at(s);
      cnt = c.cnt;
      th = terms ? exp2f((float)((double)Cu * (double)c2 - (double)c.o) - 0.00390625f) : Cu;
    }
    const int inc = wave_incl_scan_i(cnt, lane);
    const int tot = lane63(inc);
    const int pre = inc - cnt;  // list start of chunk s0 + lane
    wave_sync();
    ws.pre[lane] = pre;
    ws.thr[lane] = th;
    wave_sync();
    const int nb = min(kWave, S - s0);
    // The chunk of list position fi is the last non-empty chunk whose list
    // starts at or before fi.  Non-empty chunks start at distinct positions,
    // so with a bitmap of those starts the chunk's rank among the non-empty
    // ones is a popcount, and a table maps the rank to the chunk.  The
    // bitmap (ws.hm) and the table (ws.hc) borrow the histogram arrays,
    // which every selection clears before use.
    const bool nonempty = lane < nb && cnt > 0;
    const uint64_t neb = __ballot(nonempty);
    const int nne = __popcll(neb);
    if (nonempty) ws.hc[__popcll(neb & below)] = (uint32_t)lane;
    for (int f0 = 0; f0 < tot; f0 += kBatch * kWave) {
      int2 ent[kBatch];
      int ch[kBatch];
      if (lane < kBatch) ws.hm[lane] = 0ull;
      wave_sync();
      const int rel = pre - f0;
      if (nonempty && rel >= 0 && rel < kBatch * kWave) atomicOr(&ws.hm[rel >> 6], 1ull << (rel & 63));
      wave_sync();
      int base = __popcll(__ballot(nonempty && pre < f0)) - 1;  // rank of the chunk holding f0 - 1
#pragma unroll
      for (int q = 0; q < kBatch; ++q) {
        const unsigned long long wq = ws.hm[q];
        // (readfirstlane returns int: go through uint32_t, or the low word
        // would be sign-extended)
        const uint64_t word = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(wq >> 32)) << 32) |
                              (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)wq);
        // set bits of the word at positions <= lane: those below it (mbcnt
        // counts a scalar mask's bits below the lane) plus the lane's own
        const int below_n = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(word >> 32),
                                                           __builtin_amdgcn_mbcnt_lo((uint32_t)word, 0u));
        const int r = base + below_n + (int)((word >> lane) & 1ull);
        ch[q] = (int)ws.hc[max(0, min(r, nne - 1))];
        base += __popcll(word);
      }
#pragma unroll
      for (int q = 0; q < kBatch; ++q) {
        const int fi = f0 + q * kWave + lane;
        ent[q] = make_int2(0, 0);
        if (fi < tot) ent[q] = P.cent[(slot0 + s0 + ch[q]) * (size_t)P.cap + min(fi - ws.pre[ch[q]], P.cap - 1)];
      }
      float th[kBatch];
#pragma unroll
      for (int q = 0; q < kBatch; ++q) th[q] = ws.thr[ch[q]];
#pragma unroll
      for (int q = 0; q < kBatch; ++q) {
        const bool pass = f0 + q * kWave + lane < tot && __int_as_float(ent[q].y) >= th[q];
        const uint64_t bal = __ballot(pass);
        if (pass) {
          const int pos = nv + __popcll(bal & below);
          if (pos < kVecList) {
            ws.vi[pos] = ent[q].x;
            if (keep_keys) ws.cx[pos] = __int_as_float(ent[q].y);  // kRowCache >= kVecList
          }
        }
        nv += __popcll(bal);
      }
    }
    wave_sync();
  }
  return nv;
}

// Loads candidate vectors ws.vi[j0 + q * 64 + lane] (< nv) into registers.
template <int DT, bool VEC>
__device__ __forceinline__ void load_candidates(const KParams& P, const char* row, int j0, int nv, int lane,
                                                const WaveSmem& ws, uint4 (&v)[4], int (&e0)[4]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int j = j0 + q * kWave + lane;
    e0[q] = j < nv ? ws.vi[j] : 0;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    v[q] = make_uint4(0, 0, 0, 0);
    if (j0 + q * kWave + lane < nv) v[q] = load_vec<DT, VEC>(row, e0[q], P.V);
  }
}

// Appends the logits >= c of one vector per lane to (dx, di) at *n, in
// (lane, element) order; entries beyond cap are counted but not stored.
template <int DT>
__device__ __forceinline__ void append_ge(bool have, const uint4& v, int e0, float c, int lane, float* dx, int* di,
                                          int cap, int* n) {
  constexpr int VE = Fmt<DT>::VE;
  const uint64_t below = (1ull << lane) - 1ull;
  bool pass[VE];
  int before = 0, total = 0;
#pragma unroll
  for (int k = 0; k < VE; ++k) {
    pass[k] = have && elem<DT>(v, k) >= c;
    const uint64_t bal = __ballot(pass[k]);
    before += __popcll(bal & below);  // passing logits of the lower lanes
    total += __popcll(bal);
  }
  int pos = *n + before;
#pragma unroll
  for (int k = 0; k < VE; ++k) {
    if (pass[k]) {
      if (pos < cap) {
        dx[pos] = elem<DT>(v, k);
        di[pos] = e0 + k;
      }
      ++pos;
    }
  }
  *n += total;
}

// Merges logit row r of sequence b into sm.rows[r] (one wave).
template <int DT, bool VEC>
__device__ __forceinline__ void merge_row(const KParams& P, const SeqParams& sp, int b, int r, int lane,
                                          WaveSmem& ws, RowRec& out) {
  const int S = P.S;
  bool tgt;
  int t;
  const bool used = decode_row(P, sp, r, &tgt, &t);
  RowRec rr;
  rr.M = -kInf;
  rr.T = -kInf;
  rr.c2 = (double)(float)sp.c2;
  rr.Zs = 1.0;
  rr.pid = __builtin_nan("");
  rr.g = -1;
  rr.n_keep = -1;
  rr.flags = 0;
  rr.pad = 0;
  if (!used) {
    if (lane == 0) out = rr;
    return;
  }
  const void* row = row_ptr<DT>(P, b, tgt, t);
  const size_t rowid = (size_t)b * P.R + r;
  const size_t slot0 = rowid * S;
  const int mode = sp.mode;
  const float c2 = (float)sp.c2;
  const int tok = t < sp.Kb ? P.tokens[(size_t)b * P.K_max + t] : INT32_MIN;
  const bool tok_ok = tok != INT32_MIN && tok >= 0 && tok < P.V;
  const float xtok = tok_ok ? load_logit<DT>(row, tok) : 0.0f;  // issued early

  // chunk records: held in registers when the row has at most 64 chunks
  const ChunkRec* crec = P.chunks + slot0;
  const bool small = S <= kWave;
  ChunkRec mine;
  mine.m = -kInf;
  mine.cut = -kInf;
  mine.z = 0.0;
  mine.cnt = 0;
  mine.arg = 0x7fffffff;
  mine.flags = 0;
  mine.o = 0.0f;
  if (small && lane < S) mine = crec[lane];
  auto recs = [&](auto&& f) {
    if (small) {
      if (lane < S) f(mine);
    } else {
      for (int s = lane; s < S; s += kWave) f(crec[s]);
    }
  };
  float mx = -kInf;
  uint32_t fl = 0;
  recs([&](const ChunkRec& c) {
    mx = fmaxf(mx, c.m);
    fl |= c.flags;
  });
  const float M = wave_max(mx);
  fl = wave_or_u(fl);
  rr.M = M;
  if ((fl & kCfNonFinite) || !(M < kInf) || isnan(M)) rr.flags |= SV_ST_NONFINITE;
  else if (M == -kInf) rr.flags |= SV_ST_EMPTY;

  double Z = 0.0;
  if (!(rr.flags & kErrBits) && (mode == SV_PLAIN || mode == SV_TOPP)) {
    double term = 0.0;
    recs([&](const ChunkRec& c) {
      if (c.m > -kInf) term += c.z * exp2(((double)c.m - (double)M) * (double)c2);
    });
    Z = wave_sum(term);
    if (!(Z > 0.0) || !(Z < 1e300)) rr.flags |= SV_ST_NONFINITE;
  }

  const float oM = M * c2;
  const double fM = exp2_small((double)oM - (double)M * (double)c2);
  bool list_ok = false;
  int src = 0;  // where the candidates >= the final cut lie: 1 registers, 2 LDS cache
  int n = 0, nv = 0;
  uint4 rv[4];  // candidate vectors held in registers (src 1)
  int re[4];
  if (!(rr.flags & kErrBits)) {
    if (mode == SV_PLAIN) {
      rr.Zs = Z;
    } else if (mode == SV_GREEDY) {
      int best = 0x7fffffff;
      recs([&](const ChunkRec& c) {
        if (c.m == M) best = min(best, c.arg);
      });
      rr.g = wave_min_i(best);
      rr.T = M;
      rr.n_keep = 1;
    } else {
      // every logit >= C of the row lies in a listed candidate vector
      float cm = -kInf;
      recs([&](const ChunkRec& c) { cm = fmaxf(cm, c.cut); });
      const float C = wave_max(cm);
      const bool by_mass = mode == SV_TOPP;
      unsigned long long target;
      if (by_mass) {
        const double tt = (double)sp.topp * Z * kFix;
        target = tt < 1.0 ? 1ull : (unsigned long long)tt;
      } else {
        target = (unsigned long long)sp.topk;
      }
      const char* rowc = static_cast<const char*>(row);
      auto rec_at = [&](int s) { return small ? mine : crec[s]; };  // s = lane when small
      // A nucleus first tries the cut 8 log2 units below the row maximum
      // (its lists reach 10), then C.  The candidates >= the cut are held
      // in registers (up to 256 vectors) or cached in LDS; the full row is
      // re-read when they do not fit or the threshold falls below C.
      SelOut so;
      bool ok = false;
      // an upper bound of every logit of the row: M comes from the chunks'
      // largest terms, within a few ulps of the largest logit
      const float Mhi = M + (fabsf(M) + 1.0f) * 0.001953125f;
      float C1 = by_mass ? fmaxf(C, (float)((double)M - 8.0 / (double)c2)) : C;
      if (!by_mass && C < kInf) {
        // top-k: the k-th largest logit is at least the k-th largest vector
        // maximum (every vector holds its maximum), so that key bounds it
        const int nk0 = min(filter_listed(P, slot0, rec_at, C, c2, false, lane, ws, true), kVecList);
        const SelOut sk = select_bounded<DT>(
            [&](auto&& f) {
              for (int j = lane; j < nk0; j += kWave) f(ws.cx[j], 0ull);
            },
            false, target, ws, lane, C, Mhi);
        if (sk.reached) C1 = fmaxf(C, sk.T);
      }
      for (int pass = 0; pass < 2 && !ok && C < kInf; ++pass) {
        const float Cu = pass == 0 ? C1 : C;
        if (pass == 1 && !(C1 > C)) break;
        const float Cuf = fmaxf(Cu, -kMaxFinite);  // -inf padding never passes
        nv = filter_listed(P, slot0, rec_at, Cu, c2, by_mass, lane, ws);
        src = 0;
        if (nv <= 4 * kWave) {
          load_candidates<DT, VEC>(P, rowc, 0, nv, lane, ws, rv, re);
          so = select_bounded<DT>(
              [&](auto&& f) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                  const bool have = q * kWave + lane < nv;
                  if (__ballot(have)) {
#pragma unroll
                    for (int k = 0; k < Fmt<DT>::VE; ++k) {
                      const float x = elem<DT>(rv[q], k);
                      if (have && x >= Cuf) f(x, mass_of(x, c2, oM, fM));
                    }
                  }
                }
              },
              by_mass, target, ws, lane, Cuf, Mhi);
          src = 1;
        } else if (nv <= kVecList) {
          n = 0;
          for (int j0 = 0; j0 < nv; j0 += 4 * kWave) {
            load_candidates<DT, VEC>(P, rowc, j0, nv, lane, ws, rv, re);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const bool have = j0 + q * kWave + lane < nv;
              if (__ballot(have)) append_ge<DT>(have, rv[q], re[q], Cuf, lane, ws.cx, ws.ci, kRowCache, &n);
            }
          }
          if (n <= kRowCache) {
            wave_sync();
            so = select_bounded<DT>(
                [&](auto&& f) {
                  for (int j = lane; j < n; j += kWave) {
                    const float x = ws.cx[j];
                    f(x, mass_of(x, c2, oM, fM));
                  }
                },
                by_mass, target, ws, lane, Cuf, Mhi);
            src = 2;
          }
        }
        ok = src != 0 && so.reached && so.T >= Cu;
      }
      if (!ok) {
        // full-row selection: re-read the row
        src = 0;
        so = wave_select<DT>(
            [&](auto&& f) {
              for (int e = lane; e < P.V; e += kWave) {
                const float x = load_logit<DT>(row, e);
                f(x, mass_of(x, c2, oM, fM));
              }
            },
            by_mass, target, ws, lane);
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
      list_ok = ok && tgt && so.n_keep <= (uint32_t)kListMax;
    }
  }

  if (tok != INT32_MIN) {  // this row scores a draft token
    if (!tok_ok) {
      rr.flags |= SV_ST_TOKEN;
    } else if (!(rr.flags & kErrBits)) {
      if (mode == SV_GREEDY) rr.pid = tok == rr.g ? 1.0 : 0.0;
      else rr.pid = xtok >= rr.T ? exp2(((double)xtok - (double)M) * (double)c2) / rr.Zs : 0.0;
    }
  }

  if (list_ok && !(rr.flags & kErrBits)) {
    // the kept set, in vocabulary order: the candidates >= T, compacted in
    // list order
    rr.flags |= kRfListOk;
    int nk = 0;
    const uint64_t below = (1ull << lane) - 1ull;
    wave_sync();
    if (src == 1) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bool have = q * kWave + lane < nv;
        if (__ballot(have)) append_ge<DT>(have, rv[q], re[q], rr.T, lane, ws.cx, ws.ci, kListMax, &nk);
      }
    } else {
      for (int j0 = 0; j0 < n; j0 += kWave) {
        const int j = j0 + lane;
        const float x = j < n ? ws.cx[j] : -kInf;
        const int ix = j < n ? ws.ci[j] : 0;
        const bool keep = j < n && x >= rr.T;
        const uint64_t bal = __ballot(keep);
        wave_sync();
        if (keep) {
          const int pos = nk + __popcll(bal & below);  // pos <= j: no entry is overwritten unread
          ws.cx[pos] = x;
          ws.ci[pos] = ix;
        }
        nk += __popcll(bal);
        wave_sync();
      }
    }
    wave_sync();
    if (P.R <= kSeqWaves) {
      // the set stays in this wave's LDS for the draw, with the draft's
      // logits at its tokens (for a resample at this position)
      if (t < sp.Kb) {
        const void* drow = row_ptr<DT>(P, b, false, t);
        for (int j = lane; j < nk; j += kWave) ws.vi[j] = __float_as_int(load_logit<DT>(drow, ws.ci[j]));
      }
    } else {
      KeptEntry* kl = P.kept + rowid * (size_t)min(kListMax, P.V);  // n_keep <= min(kListMax, V)
      for (int j = lane; j < nk; j += kWave) {
        KeptEntry ke;
        ke.idx = ws.ci[j];
        ke.pad = 0;
        ke.q = (double)mass_of(ws.cx[j], c2, oM, fM) / kFix / rr.Zs;
        kl[j] = ke;
      }
    }
  }
  if (lane == 0) out = rr;
}

// ------------------------------------------------------------- draws ----

struct Draw {
  int y;
  uint32_t flags;
};

__device__ __forceinline__ int seq_min_i(int v, SmemSeq& sm) {
  v = wave_min_i(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sm.ri[threadIdx.x >> 6] = v;
  __syncthreads();
  int s = sm.ri[0];
#pragma unroll
  for (int w = 1; w < kSeqWaves; ++w) s = min(s, sm.ri[w]);
  return s;
}
__device__ __forceinline__ int seq_max_i(int v, SmemSeq& sm) {
  v = wave_max_i(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sm.ri[threadIdx.x >> 6] = v;
  __syncthreads();
  int s = sm.ri[0];
#pragma unroll
  for (int w = 1; w < kSeqWaves; ++w) s = max(s, sm.ri[w]);
  return s;
}
// Exclusive prefix over the work-group in thread order; *total = the sum.
__device__ __forceinline__ double seq_exclusive_scan(double v, double* total, SmemSeq& sm) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const double inc = wave_incl_scan(v, lane);
  __syncthreads();
  if (lane == 63) sm.rd[w] = inc;
  __syncthreads();
  double base = 0.0, tot = 0.0;
#pragma unroll
  for (int j = 0; j < kSeqWaves; ++j) {
    base += j < w ? sm.rd[j] : 0.0;
    tot += sm.rd[j];
  }
  *total = tot;
  return base + inc - v;
}

// Probability of a logit under one row's filtered distribution, with the
// terms computed as for the kept masses (mass_of): 2^(x c2 - oM) fM / Zs.
// fp32 weights (relative error ~1e-7, far inside the 1e-6 decision window),
// summed in fp64.
struct RowW {
  float c2, oM, T, sc;  // sc = fM / Zs
};
__device__ __forceinline__ RowW row_w(const RowRec& r) {
  RowW w;
  w.c2 = (float)r.c2;
  w.oM = r.M * w.c2;
  w.sc = (float)(exp2_small((double)w.oM - (double)r.M * (double)w.c2) / r.Zs);
  w.T = r.T;
  return w;
}
__device__ __forceinline__ float prob(const RowW& w, float x) {
  return x >= w.T ? __builtin_amdgcn_exp2f(fmaf(x, w.c2, -w.oM)) * w.sc : 0.0f;
}

// Inverse CDF over the target's kept set in vocabulary order (one wave):
// w = (q - p)+ when resampling, else w = q.  Entry i sits in slot i / 64 of
// lane i % 64, so a set of up to 64 tokens costs one wave step per stage.
// The set is read from the LDS of the wave that merged the row (ls), or
// from global memory.  The draft's weights are fp32 terms as in prob().
template <int DT>
__device__ __forceinline__ Draw draw_from_list(const KParams& P, const RowRec& rq, bool resample, const RowRec& rp,
                                               size_t rowq, const void* drow, double u, int lane,
                                               const WaveSmem* ls) {
  constexpr int E = kListMax / kWave;
  const int N = rq.n_keep;  // <= kListMax
  const int ns = (N + kWave - 1) / kWave;
  const RowW wp = row_w(rp);
  double qv[E];
  float pv[E];
  int iv[E];
  if (ls) {
    const float c2q = (float)rq.c2;
    const float oM = rq.M * c2q;
    const double fM = exp2_small((double)oM - (double)rq.M * (double)c2q);
    const double inv = 1.0 / (rq.Zs * kFix);
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const int i = j * kWave + lane;
      qv[j] = 0.0;
      pv[j] = 0.0f;
      iv[j] = 0;
      if (j < ns && i < N) {
        iv[j] = ls->ci[i];
        qv[j] = (double)mass_of(ls->cx[i], c2q, oM, fM) * inv;
        if (resample) pv[j] = prob(wp, __int_as_float(ls->vi[i]));
      }
    }
  } else {
    const KeptEntry* kl = P.kept + rowq * (size_t)min(kListMax, P.V);
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const int i = j * kWave + lane;
      qv[j] = 0.0;
      pv[j] = 0.0f;
      iv[j] = 0;
      if (j < ns && i < N) {
        const KeptEntry ke = kl[i];
        qv[j] = ke.q;
        iv[j] = ke.idx;
      }
    }
    if (resample) {
#pragma unroll
      for (int j = 0; j < E; ++j)
        if (j < ns && j * kWave + lane < N) pv[j] = prob(wp, load_logit<DT>(drow, iv[j]));
    }
  }
  Draw d;
  d.flags = 0;
  double w[E], ex[E];
  bool use_p = resample;
  double total = 0.0;
  for (int pass = 0; pass < 2; ++pass) {
    total = 0.0;  // running sum in vocabulary order: slot by slot, lanes in order
#pragma unroll
    for (int j = 0; j < E; ++j) {
      w[j] = 0.0;
      ex[j] = total;
      if (j < ns) {
        w[j] = use_p ? fmax(qv[j] - (double)pv[j], 0.0) : qv[j];
        const double inc = wave_incl_scan(w[j], lane);
        ex[j] = total + (inc - w[j]);
        total += lane63(inc);
      }
    }
    if (total > 0.0 || !use_p) break;
    d.flags |= SV_ST_ZERO_RESIDUAL;  // (q - p)+ has no mass: draw from q
    use_p = false;
  }
  const double target = u * total;
  // first entry whose running sum exceeds the target; the last non-zero one
  int first = 0x7fffffff, lastnz = -1, firstnz = 0x7fffffff;
  double clo = 0.0, chi = 0.0;
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const int i = j * kWave + lane;
    const double cn = ex[j] + w[j];
    if (j < ns && i < N && w[j] > 0.0) {
      if (cn > target && first == 0x7fffffff) {
        first = i;
        clo = ex[j];
        chi = cn;
      }
      lastnz = max(lastnz, i);
      firstnz = min(firstnz, i);
    }
  }
  const int f = wave_min_i(first);
  const int lnz = wave_max_i(lastnz);
  const int fnz = wave_min_i(firstnz);
  int iy;
  double lo, hi;
  if (f <= lnz) {
    iy = f;
    lo = lane_at(clo, f % kWave);
    hi = lane_at(chi, f % kWave);
  } else {  // rounding left no entry above the target
    iy = lnz < 0 ? 0 : lnz;
    lo = total;
    hi = total;
  }
  int yv = 0;
#pragma unroll
  for (int j = 0; j < E; ++j)
    if (j * kWave + lane == iy) yv = iv[j];
  d.y = N > 0 ? lane_at(yv, iy % kWave) : 0;
  if (N > 0 && lnz >= 0 && total > 0.0) {
    // margins of interior CDF boundaries
    if ((fnz < iy && u - lo / total < kWindow) || (lnz > iy && hi / total - u < kWindow)) d.flags |= SV_ST_MARGIN;
  }
  return d;
}

// Raw logits of the 8 tokens e..e+7 of one row, in 1 (bf16) or 2 (fp32)
// 16-byte vectors (-inf past V).
template <int DT, bool VEC>
__device__ __forceinline__ void load8(const KParams& P, const char* row, int e, uint4 (&r)[2]) {
  constexpr int VE = Fmt<DT>::VE;
  const uint32_t ninf = DT == SV_BF16 ? 0xff80ff80u : 0xff800000u;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    r[h] = make_uint4(ninf, ninf, ninf, ninf);
    if (h * VE < 8 && e + h * VE < P.V) r[h] = load_vec<DT, VEC>(row, e + h * VE, P.V);  // whole vectors when VEC
  }
}

// prob() for a row that keeps every token (threshold -inf): the kept-set
// test always passes, since a row a draw reads holds no NaN (a NaN makes the
// sequence an error row before any draw), and -inf still weighs 0.
__device__ __forceinline__ float prob_all(const RowW& w, float x) {
  return __builtin_amdgcn_exp2f(fmaf(x, w.c2, -w.oM)) * w.sc;
}

// Weights of 8 tokens in fp32: q, or (q - p)+; returns their sum, added
// pairwise in fp32 (both passes of a row draw use this same group sum).
// Tokens past the row end were loaded as -inf and weigh 0, and a walked
// range never ends inside a group of 8 except at the row end, so no bound
// test is needed.  `all` (wave-uniform): every row read keeps every token,
// so the threshold test is left out.
template <int DT>
__device__ __forceinline__ float weights8(const RowW& wq, bool use_p, const RowW& wp, bool all,
                                          const uint4 (&rq)[2], const uint4 (&rp)[2], float (&w)[8]) {
  constexpr int VE = Fmt<DT>::VE;
  if (all) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      float q = prob_all(wq, elem<DT>(rq[k / VE], k % VE));
      if (use_p) q = fmaxf(q - prob_all(wp, elem<DT>(rp[k / VE], k % VE)), 0.0f);
      w[k] = q;
    }
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      float q = prob(wq, elem<DT>(rq[k / VE], k % VE));
      if (use_p) q = fmaxf(q - prob(wp, elem<DT>(rp[k / VE], k % VE)), 0.0f);
      w[k] = q;
    }
  }
  return ((w[0] + w[1]) + (w[2] + w[3])) + ((w[4] + w[5]) + (w[6] + w[7]));
}

// Inverse CDF over logit rows re-read from memory by the whole work-group.
// The range [lo, hi) (the whole row, or for a plain bonus draw the chunk
// that the chunk records place the target in) is split into one segment
// per wave; pass 1 sums the weights of each 512-token tile into LDS, pass 2
// scans the one tile that holds the target.
template <int DT, bool VEC>
__device__ __forceinline__ Draw draw_from_rows(const KParams& P, const RowRec& rq, bool resample, const RowRec& rp,
                                               const char* qrow, const char* prow, double u, SmemSeq& sm, int lane,
                                               int wv, const ChunkRec* qrec) {
  constexpr int kTileCap = (int)(kRowCache * sizeof(float) / sizeof(double));
  const int tid = threadIdx.x;
  Draw d;
  d.flags = SV_ST_REREAD;
  d.y = 0;
  const RowW wq = row_w(rq), wp = row_w(rp);
  bool use_p = resample;
  const bool all = __builtin_amdgcn_readfirstlane((int)(wq.T == -kInf && (!resample || wp.T == -kInf))) != 0;
  int lo = 0, hi = P.V;
  double base = 0.0;  // weight before lo (chunk-located draws)
  bool located = false, force_last = false;
  if (!resample && qrec && rq.T == -kInf) {
    // plain bonus draw: the chunk sums give the chunk holding u
    const int S = P.S;
    // two chunks per thread cover every row: V <= 2^22 is at most 1024 chunks
    static_assert(2 * kSeqThreads >= kMaxVocab / (64 * kLoads * 4), "chunk sums per thread");
    double wc[2];
    for (int j = 0; j < 2; ++j) {
      const int c = 2 * tid + j;
      wc[j] = 0.0;
      if (c < S) {
        const ChunkRec r = qrec[c];
        if (r.m > -kInf) wc[j] = r.z * exp2(((double)r.m - (double)rq.M) * (double)wq.c2) / rq.Zs;
      }
    }
    double tot;
    const double ex = seq_exclusive_scan(wc[0] + wc[1], &tot, sm);
    int cstar = 0x7fffffff, clast = -1;
    double cb = 0.0;
    for (int j = 0; j < 2; ++j) {
      const int c = 2 * tid + j;
      const double before = ex + (j ? wc[0] : 0.0);
      if (c < S && wc[j] > 0.0) {
        if (before + wc[j] > u && cstar == 0x7fffffff) {
          cstar = c;
          cb = before;
        }
        clast = c;
      }
    }
    const int cs = seq_min_i(cstar, sm);
    const int cl = seq_max_i(clast, sm);
    if (cs != 0x7fffffff || cl >= 0) {
      const int c = cs != 0x7fffffff ? cs : cl;
      __syncthreads();
      if (cs != 0x7fffffff ? (cstar == cs) : false) sm.rd[0] = cb;
      __syncthreads();
      base = cs != 0x7fffffff ? sm.rd[0] : 0.0;
      __syncthreads();
      lo = c * P.L;
      hi = min(P.V, lo + P.L);
      located = true;
      force_last = cs == 0x7fffffff;  // u beyond the rounded total: the last token of the last chunk
    }
  }
  double* tsum = reinterpret_cast<double*>(sm.w[wv].cx);  // this wave's tile sums
  double S = 0.0;
  int nzlo = 0x7fffffff, nzhi = -1, per = 0, v0 = 0, v1 = 0;
  for (int pass = 0; pass < 2; ++pass) {
    const int n8 = (hi - lo + 7) / 8;
    per = (n8 + kSeqWaves - 1) / kSeqWaves;
    v0 = min(n8, wv * per);
    v1 = min(n8, v0 + per);
    double seg = 0.0;
    int zl = 0x7fffffff, zh = -1, nt = 0;
    for (int t0 = v0; t0 < v1; t0 += kDrawTiles * kWave) {
      // the loads of kDrawTiles tiles are in flight together
      uint4 rq[kDrawTiles][2], rp[kDrawTiles][2];
#pragma unroll
      for (int g = 0; g < kDrawTiles; ++g) {
        const int vi = t0 + g * kWave + lane;
        const uint32_t ninf = DT == SV_BF16 ? 0xff80ff80u : 0xff800000u;
        rq[g][0] = rq[g][1] = rp[g][0] = rp[g][1] = make_uint4(ninf, ninf, ninf, ninf);
        if (vi < v1) {
          load8<DT, VEC>(P, qrow, lo + 8 * vi, rq[g]);
          if (use_p) load8<DT, VEC>(P, prow, lo + 8 * vi, rp[g]);
        }
      }
#pragma unroll
      for (int g = 0; g < kDrawTiles; ++g) {
        if (t0 + g * kWave >= v1) break;
        const int vi = t0 + g * kWave + lane;
        double sl = 0.0;
        if (vi < v1) {
          float w[8];
          const float s8 = weights8<DT>(wq, use_p, wp, all, rq[g], rp[g], w);
          sl = (double)s8;
          // the first and last groups of 8 with weight (refined to a token
          // only where that is needed)
          if (s8 > 0.0f) {
            zl = min(zl, lo + 8 * vi);
            zh = max(zh, lo + 8 * vi + 7);
          }
        }
        sl = wave_sum(sl);
        if (lane == 0 && nt < kTileCap) tsum[nt] = sl;
        seg += sl;
        ++nt;
      }
    }
    zl = wave_min_i(zl);
    zh = wave_max_i(zh);
    __syncthreads();
    if (lane == 0) {
      sm.rd[wv] = seg;
      sm.ri[wv] = zl;
    }
    __syncthreads();
    S = 0.0;
    nzlo = 0x7fffffff;
#pragma unroll
    for (int w = 0; w < kSeqWaves; ++w) {
      S += sm.rd[w];
      nzlo = min(nzlo, sm.ri[w]);
    }
    __syncthreads();
    if (lane == 0) sm.ri[wv] = zh;
    __syncthreads();
    nzhi = -1;
#pragma unroll
    for (int w = 0; w < kSeqWaves; ++w) nzhi = max(nzhi, sm.ri[w]);
    if (!(S > 0.0) && use_p) {
      d.flags |= SV_ST_ZERO_RESIDUAL;  // (q - p)+ has no mass: draw from q
      use_p = false;
      __syncthreads();
      continue;
    }
    break;
  }
  // the target: u * S over the whole row, or u - base within the located chunk
  const double target = located ? (force_last ? kInf : u - base) : u * S;
  // the wave segment, then the tile, holding the target
  int ws_ = -1;
  double before = 0.0;
  {
    double c = 0.0;
    for (int w = 0; w < kSeqWaves; ++w) {
      const double sw = sm.rd[w];
      if (ws_ < 0 && sw > 0.0 && c + sw > target) {
        ws_ = w;
        before = c;
      }
      c += sw;
    }
  }
  int y = -1;
  double clo = 0.0, chi = 0.0;
  if (ws_ >= 0 && wv == ws_) {
    const int n8 = (hi - lo + 7) / 8;
    const int a0 = min(n8, ws_ * per), a1 = min(n8, a0 + per);
    int t = 0;
    double c = before;
    const int ntile = (a1 - a0 + kWave - 1) / kWave;
    if (ntile <= kTileCap) {
      while (t < ntile - 1 && !(tsum[t] > 0.0 && c + tsum[t] > target)) c += tsum[t++];
    }
    // scan tiles from t (usually just one) until the target is crossed
    for (; t < ntile && y < 0; ++t) {
      const int vi = a0 + t * kWave + lane;
      double w[8];
      double sl = 0.0;
      if (vi < a1) {
        uint4 aq[2], ap[2];
        const uint32_t ninf = DT == SV_BF16 ? 0xff80ff80u : 0xff800000u;
        ap[0] = ap[1] = make_uint4(ninf, ninf, ninf, ninf);
        load8<DT, VEC>(P, qrow, lo + 8 * vi, aq);
        if (use_p) load8<DT, VEC>(P, prow, lo + 8 * vi, ap);
        float wf[8];
        sl = (double)weights8<DT>(wq, use_p, wp, all, aq, ap, wf);
#pragma unroll
        for (int k = 0; k < 8; ++k) w[k] = (double)wf[k];
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) w[k] = 0.0;
      }
      const double inc = wave_incl_scan(sl, lane);
      const double tile = lane63(inc);
      if (c + tile > target) {
        int cand = 0x7fffffff;
        double r = c + inc - sl, cl = 0.0, ch = 0.0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const double rn = r + w[k];
          if (rn > target && w[k] > 0.0 && cand == 0x7fffffff) {
            cand = lo + 8 * vi + k;
            cl = r;
            ch = rn;
          }
          r = rn;
        }
        const int ym = wave_min_i(cand);
        if (ym != 0x7fffffff) {
          const uint64_t who = __ballot(cand == ym);
          const int src = __ffsll((long long)who) - 1;
          y = ym;
          clo = lane_at(cl, src);
          chi = lane_at(ch, src);
        }
      }
      c += tile;
    }
    if (lane == 0) {
      sm.misc[2] = (uint32_t)y;
      sm.rx[0] = clo;
      sm.rx[1] = chi;
    }
  }
  __syncthreads();
  if (ws_ >= 0) {
    y = (int)sm.misc[2];
    clo = sm.rx[0];
    chi = sm.rx[1];
  }
  __syncthreads();
  if (y < 0) {  // rounding left no token above the target: the last token with weight
    y = 0;
    if (nzhi >= 0) {
      const int g0 = nzhi - 7;  // the last group of 8 with weight
      uint4 aq[2], ap[2];
      const uint32_t ninf = DT == SV_BF16 ? 0xff80ff80u : 0xff800000u;
      ap[0] = ap[1] = make_uint4(ninf, ninf, ninf, ninf);
      load8<DT, VEC>(P, qrow, g0, aq);
      if (use_p) load8<DT, VEC>(P, prow, g0, ap);
      float wf[8];
      (void)weights8<DT>(wq, use_p, wp, all, aq, ap, wf);
      y = g0;
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (wf[k] > 0.0f) y = g0 + k;
    }
    clo = chi = S;
  }
  d.y = y;
  // the CDF just below and at y, in probability units
  const double plo = located ? base + clo : clo / S, phi = located ? base + chi : chi / S;
  if (nzlo < y && u - plo < kWindow) d.flags |= SV_ST_MARGIN;
  if (nzhi > y && phi - u < kWindow) d.flags |= SV_ST_MARGIN;
  return d;
}

// An error row: accepted = -1, every token -1, diagnostics NaN (threads
// first, first + stride, ... of the caller's group).
__device__ __forceinline__ void write_error(const KParams& P, int b, uint32_t st, int first, int stride) {
  for (int i = first; i <= P.K_max; i += stride) P.out_tokens[(size_t)b * (P.K_max + 1) + i] = -1;
  if (P.diag)
    for (int i = first; i < 2 * P.K_max; i += stride) P.diag[(size_t)b * 2 * P.K_max + i] = __builtin_nanf("");
  if (first == 0) {
    P.accepted[b] = -1;
    if (P.status) P.status[b] = st;
  }
}

// Accepted drafts d_0..d_{n-1}, then y, then -1 (threads first, first +
// stride, ...).
__device__ __forceinline__ void write_tokens(const KParams& P, int b, int n, int y, uint32_t st, int first,
                                             int stride) {
  const int KM = P.K_max;
  for (int i = first; i <= KM; i += stride) {
    int val = -1;
    if (i < n) val = P.tokens[(size_t)b * KM + i];
    else if (i == n) val = y;
    P.out_tokens[(size_t)b * (KM + 1) + i] = val;
  }
  if (first == 0) {
    P.accepted[b] = n;
    if (P.status) P.status[b] = st & ~kRfListOk;
  }
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kSeqThreads) void seq_kernel(const KParams P) {
  __shared__ SmemSeq sm;
  const int tid = threadIdx.x, lane = (int)__lane_id();
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  const int b = P.b_base + (int)blockIdx.x;
  const SeqParams sp = load_params(P, b);
  if (!sp.valid) {
    write_error(P, b, SV_ST_PARAM, tid, kSeqThreads);
    return;
  }
  const int Kb = sp.Kb, KM = P.K_max, R = P.R;
  const uint64_t g = P.row_offset + (uint64_t)b;
  // With fewer rows than waves the last wave is free during the merge: it
  // draws the walk's uniforms (they depend only on seed, sequence, position
  // and purpose), which takes them off the path after the barrier.
  const bool pre_u = R < kSeqWaves;
  for (int r = wv; r < R; r += kSeqWaves) merge_row<DT, VEC>(P, sp, b, r, lane, sm.w[wv], sm.rows[r]);
  if (pre_u && wv == kSeqWaves - 1) {
    const int t = lane;
    if (t < Kb) sm.ua[t] = uniform24(P.seed, g, (uint32_t)t, kPurposeAccept);
    if (t <= Kb) sm.ud[t] = uniform24(P.seed, g, (uint32_t)t, t < Kb ? kPurposeResample : kPurposeBonus);
  }
  __syncthreads();

  // Wave 0: the rows' flags, the accept walk, and the draw when it needs no
  // more than the kept set in LDS.  The work-group joins only for a draw
  // from the rows.
  if (wv == 0) {
    uint32_t st = 0;
    for (int t = lane; t <= Kb; t += kWave) st |= sm.rows[t].flags;
    for (int t = lane; t < Kb; t += kWave) st |= sm.rows[KM + 1 + t].flags;
    st = wave_or_u(st) & ~kRfListOk;
    int job = 0;  // 0 done, 1 draw from the rows
    if (st & kErrBits) {
      write_error(P, b, st & kErrBits, lane, kWave);
    } else {
      if (P.diag) {
        for (int t = lane; t < KM; t += kWave) {
          float q = __builtin_nanf(""), p = __builtin_nanf("");
          if (t < Kb) {
            q = (float)sm.rows[t].pid;
            p = (float)sm.rows[KM + 1 + t].pid;
          }
          P.diag[((size_t)b * KM + t) * 2 + 0] = q;
          P.diag[((size_t)b * KM + t) * 2 + 1] = p;
        }
      }
      // lane t scores position t0 + t; the first rejection by ballot.  The
      // same lanes draw the uniform of a resample at t (t < K_b) or of the
      // bonus (t = K_b), so the draw's uniform is ready with n.
      int n = Kb;
      double u = 0.0;
      for (int t0 = 0; t0 <= Kb; t0 += kWave) {
        const int t = t0 + lane;
        bool rej = false;
        uint32_t s2 = 0;
        double ud = 0.0;
        const bool have_u = pre_u && t0 == 0;  // drawn during the merge (t < 64)
        if (t < Kb) {
          const double q = sm.rows[t].pid, p = sm.rows[KM + 1 + t].pid;
          const double ua = have_u ? sm.ua[t] : uniform24(P.seed, g, (uint32_t)t, kPurposeAccept);
          rej = !(ua * p < q);
          if (p == 0.0) s2 |= SV_ST_PZERO;
          // q / p < 1 + w and |u - q / p| < w, multiplied through by p > 0
          if (p > 0.0 && q < p * (1.0 + kWindow) && fabs(ua * p - q) < kWindow * p) s2 |= SV_ST_MARGIN;
        }
        if (t <= Kb)
          ud = have_u ? sm.ud[t] : uniform24(P.seed, g, (uint32_t)t, t < Kb ? kPurposeResample : kPurposeBonus);
        const uint64_t rb = __ballot(rej);
        const int end = rb ? t0 + __ffsll((long long)rb) - 1 : Kb;  // the walk stops here if < t0 + 64
        // status bits of the positions the walk reached (up to the first rejection)
        st |= wave_or_u((t <= end && t < Kb) ? s2 : 0u);
        if (end < t0 + kWave) {
          n = end;
          u = lane_at(ud, n - t0);
          break;
        }
      }
      const bool resample = n < Kb;
      const RowRec& rq = sm.rows[n];
      const RowRec& rp = resample ? sm.rows[KM + 1 + n] : sm.rows[n];
      if (sp.mode == SV_GREEDY) {
        const int y = rq.g;
        if (resample && rp.g == rq.g) st |= SV_ST_ZERO_RESIDUAL;
        write_tokens(P, b, n, y, st, lane, kWave);
      } else if (rq.flags & kRfListOk) {
        const Draw d = draw_from_list<DT>(P, rq, resample, rp, (size_t)b * R + n,
                                          resample ? row_ptr<DT>(P, b, false, n) : nullptr, u, lane,
                                          R <= kSeqWaves ? &sm.w[n] : nullptr);
        write_tokens(P, b, n, d.y, st | d.flags, lane, kWave);
      } else {
        job = 1;
        if (lane == 0) {
          sm.misc[0] = (uint32_t)n;
          sm.misc[1] = st;
          sm.rx[0] = u;
        }
      }
    }
    if (lane == 0) sm.misc[2] = (uint32_t)job;
  }
  __syncthreads();
  if (sm.misc[2] == 0u) return;
  // draw from the rows (plain mode, or a kept set not held as a list)
  const int n = (int)sm.misc[0];
  uint32_t st = sm.misc[1];
  const double u = sm.rx[0];
  const bool resample = n < Kb;
  const RowRec rq = sm.rows[n];
  const RowRec rp = resample ? sm.rows[KM + 1 + n] : rq;
  __syncthreads();  // sm.misc / sm.rx are reused by the draw
  const Draw d = draw_from_rows<DT, VEC>(P, rq, resample, rp, static_cast<const char*>(row_ptr<DT>(P, b, true, n)),
                                         resample ? static_cast<const char*>(row_ptr<DT>(P, b, false, n)) : nullptr,
                                         u, sm, lane, wv, P.chunks + ((size_t)b * R + n) * P.S);
  write_tokens(P, b, n, d.y, st | d.flags, tid, kSeqThreads);
}

// start / stop: events recorded on the kernel's own dispatch (NULL: none).
template <int DT, bool VEC>
void launch_chunk(const KParams& p, int mode, dim3 grid, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  const dim3 block(kThreads);
  switch (mode) {
    case SV_PLAIN: hipExtLaunchKernelGGL((chunk_kernel<DT, VEC, SV_PLAIN>), grid, block, 0, stream, start, stop, 0, p); break;
    case SV_TOPK: hipExtLaunchKernelGGL((chunk_kernel<DT, VEC, SV_TOPK>), grid, block, 0, stream, start, stop, 0, p); break;
    case SV_TOPP: hipExtLaunchKernelGGL((chunk_kernel<DT, VEC, SV_TOPP>), grid, block, 0, stream, start, stop, 0, p); break;
    case SV_GREEDY: hipExtLaunchKernelGGL((chunk_kernel<DT, VEC, SV_GREEDY>), grid, block, 0, stream, start, stop, 0, p); break;
    default: hipExtLaunchKernelGGL((chunk_kernel<DT, VEC, kAnyMode>), grid, block, 0, stream, start, stop, 0, p); break;
  }
}

template <int DT, bool VEC>
hipError_t launch_all(const KParams& p, int nseq, hipStream_t stream, hipEvent_t* ev) {
  // one streaming instance: the default mode's, or the one holding every
  // path when the call gives a mode per sequence
  const size_t waves = (size_t)nseq * p.R * p.S;
  const dim3 grid((unsigned)((waves + kThreads / kWave - 1) / (kThreads / kWave)));
  launch_chunk<DT, VEC>(p, p.mode ? kAnyMode : p.dmode, grid, stream, ev ? ev[0] : nullptr, ev ? ev[1] : nullptr);
  hipExtLaunchKernelGGL((seq_kernel<DT, VEC>), dim3((unsigned)nseq), dim3(kSeqThreads), 0, stream,
                        ev ? ev[2] : nullptr, ev ? ev[3] : nullptr, 0, p);
  return hipSuccess;
}

}  // namespace

namespace {

// Read-only streaming probe with the streaming pass's access pattern and
// non-temporal loads: each wave reads one 16 KB block as 16 x 16-byte
// vectors per lane from one base address with constant offsets, and folds it
// with xor.  out[0] is written only if the fold hits a fixed value, so the
// loads cannot be dropped.
__global__ __launch_bounds__(kThreads) void stream_probe_kernel(const uint4* data, size_t nblocks, uint32_t* out) {
  const int lane = (int)__lane_id();
  const size_t blk = (size_t)blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave;
  if (blk >= nblocks) return;
  const uint4* base = data + blk * (size_t)(kLoads * kWave);
  uint4 v[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) v[i] = load_stream(&base[i * kWave + lane]);
  uint32_t x = 0;
#pragma unroll
  for (int i = 0; i < kLoads; ++i) x ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  if (x == 0x9e3779b9u) out[0] = x;
}

}  // namespace

hipError_t launch_stream_probe(const void* data, size_t bytes, uint32_t* out, hipStream_t stream) {
  const size_t nblocks = bytes / (kLoads * kWave * sizeof(uint4));
  if (nblocks == 0) return hipSuccess;
  const size_t wg = (nblocks + kThreads / kWave - 1) / (kThreads / kWave);
  hipLaunchKernelGGL(stream_probe_kernel, dim3((unsigned)wg), dim3(kThreads), 0, stream,
                     static_cast<const uint4*>(data), nblocks, out);
  return hipGetLastError();
}

hipError_t launch_verify(const KParams& p, int dtype, bool vec, int nseq, hipStream_t stream, hipEvent_t* ev) {
  if (nseq <= 0) return hipSuccess;
  hipError_t e;
  if (dtype == SV_BF16) e = vec ? launch_all<SV_BF16, true>(p, nseq, stream, ev) : launch_all<SV_BF16, false>(p, nseq, stream, ev);
  else e = vec ? launch_all<SV_F32, true>(p, nseq, stream, ev) : launch_all<SV_F32, false>(p, nseq, stream, ev);
  const hipError_t l = hipGetLastError();
  return e != hipSuccess ? e : l;
}

}  // namespace sv
