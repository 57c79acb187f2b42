// gfx950 kernels of the verify-and-resample step of speculative sampling.
//
// A call runs two kernels on the caller's stream; the kernel boundary orders
// them, so no work-group ever waits for another:
//
//   row_kernel   one work-group of 4 waves per logit row (target positions
//                0..K_b and draft positions 0..K_b-1 of every sequence).
//                The waves stream the row from HBM once, 8 KB per wave at a
//                time into registers, two chunks in flight, and reduce it:
//                the sum of the terms 2^((x - m) c2) and the maximum of
//                every chunk, the greedy argmax, and the candidate vectors
//                of a top-k / nucleus kept set, which stay in LDS.  Then the
//                whole work-group finishes the row: log-sum-exp over the
//                chunks, the threshold by radix selection over the
//                candidates, the kept mass, the probability of the row's
//                draft token and, for target rows, the kept set in
//                vocabulary order.
//   seq_kernel   one work-group per sequence: the accept walk, the first
//                rejection, the resample from normalize((q - p)+) or the
//                bonus draw, and the outputs.
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
// Nucleus candidates: tokens whose term is within 2^-10 of the largest term
// known (on the pages' workloads a window of 2^-8 to 2^-9.4 already covers
// the nucleus; a list that would overflow is compacted and retried with the
// windows 2^-8, 2^-6, 2^-5, 2^-4, 2^-3, 2^-2).
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
__device__ __forceinline__ int wave_sum_i(int v) {
  return lane63(wave_scan(v, 0, [](int a, int b) { return a + b; }));
}
__device__ __forceinline__ int wave_min_i(int v) {
  return lane63(wave_scan(v, 0x7fffffff, [](int a, int b) { return min(a, b); }));
}
__device__ __forceinline__ int wave_max_i(int v) {
  return lane63(wave_scan(v, (int)0x80000000, [](int a, int b) { return max(a, b); }));
}
// Maximum of values >= 0 (or +inf) over the wave, taken on their bit
// patterns, which such floats order as the values (no NaN handling needed).
__device__ __forceinline__ float wave_max_nonneg(float v) {
  return __int_as_float(wave_max_i(__float_as_int(v)));
}
__device__ __forceinline__ uint32_t wave_or_u(uint32_t v) {
  return lane63(wave_scan(v, 0u, [](uint32_t a, uint32_t b) { return a | b; }));
}
// How many of the lanes below this one have their bit set in the wave-uniform
// mask bal (v_mbcnt from the scalar mask; no per-lane mask register).
__device__ __forceinline__ int lanes_below(uint64_t bal) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
}

// A wave-uniform value moved to scalar registers.
__device__ __forceinline__ double uniform_d(double v) {
  return lane_at(v, 0);
}

// The lane id, opaque to the compiler: expressions of it are recomputed
// where they are used instead of being hoisted out of a loop and held in
// registers (or spilled) across it.
__device__ __forceinline__ int fresh_lane(int lane) {
  asm volatile("" : "+v"(lane));
  return lane;
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

// A load whose address is the same for the whole wave, through the scalar
// cache: its wait (lgkmcnt) is apart from that of the vector loads in
// flight, so it never waits for a chunk of logits issued before it.  Only
// for 4-byte values that the same kernel does not write (the scalar cache
// is invalidated when a kernel starts, not while it runs).
template <class T>
__device__ __forceinline__ T uniform_load(const T* p) {
  static_assert(sizeof(T) == 4, "scalar loads of 4-byte values");
  return *(const __attribute__((address_space(4))) T*)p;
}

// A load from global memory as such (not through a generic address), so
// that waiting for it never waits for the loads issued after it.
template <class T>
__device__ __forceinline__ T global_load(const T* p) {
  return *(const __attribute__((address_space(1))) T*)p;
}

// The sequence's parameters as stored (the loads only) ...  kDirect: the
// per-sequence values are loaded from global memory as such (the compiler
// takes them through the scalar cache), else through generic addresses
// (fewer scalar registers: the instance holding every mode's path).
template <bool kDirect = true>
__device__ __forceinline__ SeqParams raw_params(const KParams& P, int b, int mode) {
  SeqParams s;
  s.mode = mode;
  if constexpr (kDirect) {
    s.Kb = P.kpr ? uniform_load(P.kpr + b) : P.K_max;
    s.tau = P.temp ? global_load(P.temp + b) : P.dtemp;
    s.topk = P.topk ? global_load(P.topk + b) : P.dtopk;
    s.topp = P.topp ? global_load(P.topp + b) : P.dtopp;
  } else {
    s.Kb = P.kpr ? P.kpr[b] : P.K_max;
    s.tau = P.temp ? P.temp[b] : P.dtemp;
    s.topk = P.topk ? P.topk[b] : P.dtopk;
    s.topp = P.topp ? P.topp[b] : P.dtopp;
  }
  s.c2 = 0.0;
  s.valid = false;
  return s;
}

// ... and checked: valid, and the effective mode with c2 = log2(e) / tau.
__device__ __forceinline__ SeqParams check_params(const KParams& P, SeqParams s) {
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

__device__ __forceinline__ SeqParams load_params(const KParams& P, int b) {
  return check_params(P, raw_params(P, b, raw_mode(P, b)));
}

template <int DT>
__device__ __forceinline__ const void* row_ptr(const KParams& P, int b, bool tgt, int t) {
  constexpr int ES = Fmt<DT>::ES;
  const size_t r = tgt ? ((size_t)b * (P.K_max + 1) + t) : ((size_t)b * P.K_max + t);
  return static_cast<const char*>(tgt ? P.target : P.draft) + r * (size_t)P.V * ES;
}


// ================================================== chunk reductions ====
//
// A wave holds one chunk of a logit row in registers (64 lanes x kLoads
// vectors) and reduces it with wave ballots and DPP moves only.

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

// Makes the compiler forget what it knows of buf's values (the asm emits
// nothing): a later pass unpacks the logits again instead of keeping the
// first pass's 128 unpacked values live in registers.
__device__ __forceinline__ void unpack_barrier(uint4 (&buf)[kLoads]) {
#pragma unroll
  for (int i = 0; i < kLoads; ++i) asm volatile("" : "+v"(buf[i].x), "+v"(buf[i].y), "+v"(buf[i].z), "+v"(buf[i].w));
}

// load_chunk for a whole chunk (c1 = c0 + 64 * kLoads * VE).
template <int DT, bool VEC>
__device__ __forceinline__ void load_whole_chunk(uint4 (&buf)[kLoads], const char* row, int c0, int lane) {
  constexpr int VE = Fmt<DT>::VE, ES = Fmt<DT>::ES;
  if constexpr (VEC) {
    // one base address and constant offsets
    const uint4* base = reinterpret_cast<const uint4*>(row + (size_t)c0 * ES);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) buf[i] = load_stream(&base[i * kWave + lane]);
  } else {
    load_chunk<DT, VEC>(buf, row, c0, c0 + kWave * kLoads * VE, lane);
  }
}

// A buffer resource over one logit row of `bytes` bytes: buffer loads past
// its end return 0 instead of reading memory.  The row is the same for the
// whole wave; its address goes through readfirstlane so that the resource
// lives in scalar registers (a resource the compiler cannot prove uniform
// turns every load into a loop over the lanes' distinct values).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_resource(const char* row, int bytes) {
  const uint64_t a = reinterpret_cast<uintptr_t>(row);
  const uint64_t u = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32)) << 32) |
                     (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>((uintptr_t)u), (short)0,
                                           __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// Issues the loads of the chunk at byte offset `off` of a row of whole
// 16-byte vectors, through the row's buffer resource (non-temporal: every
// logit is read once).  The offset goes into the per-lane offset, which the
// hardware checks against the row's size: vectors past the row's end read
// as 0 without touching memory, and off = the row's size issues loads that
// all read 0 (so that a wave always has the same number of loads in flight).
// mask_chunk makes every vector past the chunk's end -inf once the data is
// needed, so that issuing the loads does not wait for them.
template <int DT>
__device__ __forceinline__ void issue_chunk(uint4 (&buf)[kLoads], __amdgpu_buffer_rsrc_t rs, int off, int lane) {
  const int v0 = off + lane * 16;
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, v0 + i * kWave * 16, 0, 2);
    buf[i] = make_uint4(v.x, v.y, v.z, v.w);
  }
}
template <int DT>
__device__ __forceinline__ void mask_chunk(uint4 (&buf)[kLoads], int c0, int c1, int lane) {
  constexpr int VE = Fmt<DT>::VE;
  const uint32_t ninf = DT == SV_BF16 ? 0xff80ff80u : 0xff800000u;
  const int nvec = (c1 - c0) / VE;
  if (nvec >= kWave * kLoads) return;  // a whole chunk (wave-uniform)
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const bool ok = i * kWave + lane < nvec;
    buf[i].x = ok ? buf[i].x : ninf;
    buf[i].y = ok ? buf[i].y : ninf;
    buf[i].z = ok ? buf[i].z : ninf;
    buf[i].w = ok ? buf[i].w : ninf;
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

// One exp per logit: returns the lane's sum of the chunk's terms
// 2^(x c2 - o), the largest term of each of its vectors (emax[i]) and its
// largest term (*em).  The exponent x c2 - o is rounded once (fma).  The
// logits are only used through the terms, so each vector is unpacked right
// where it is consumed.
template <int DT>
__device__ __forceinline__ float exp_terms(const uint4 (&buf)[kLoads], float c2, float o, float (&emax)[kLoads],
                                           float* em) {
  constexpr int VE = Fmt<DT>::VE;
  float acc = 0.0f, mx = 0.0f;
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
    mx = fmaxf(mx, mi);
    acc += si;
  }
  *em = mx;
  return acc;
}

// Lane-local softmax sums of the streaming pass (plain and nucleus rows).
// Every lane adds the terms 2^(x c2 - o) of its own logits, over all the
// chunks of its wave, into an fp64 sum, so a chunk costs no wave-wide sum.
// The offset o is wave-uniform, an integer, and only grows: raising it
// rescales the sums by a power of two, which is exact.
struct SoftAcc {
  double z;   // the lane's sum of 2^(x c2 - o)
  float o;    // the exponent offset (-inf until the wave has seen a finite logit)
  float lt;   // the largest x c2 of the wave's logits so far, from its largest term (-inf: none)
};

// Raises the offset to floor(xc2) if that is larger (and finite).
__device__ __forceinline__ void raise_offset(SoftAcc& sa, float xc2) {
  const float on = floorf(xc2);
  if (on > sa.o && on < kInf) {
    if (sa.o > -kInf) sa.z = ldexp(sa.z, (int)fmaxf(sa.o - on, -2000.0f));
    sa.o = on;
  }
}

struct SoftChunk {
  float zt;  // the lane's sum of the chunk's terms 2^(x c2 - o)
  float o;   // the offset o of those terms
  float em;  // the chunk's largest term (wave-uniform; 0 if none)
  bool ok;   // false: the chunk holds a NaN or +inf, or a logit whose x c2 overflows fp32
};

// Adds one chunk (held in buf, -inf past the row's end) to the lane sums.
// A term is rounded in its exponent x c2 - o, so it is accurate to about
// |x c2 - o| 2^-24 relative, and the largest terms, which dominate the sum,
// need o close to the maximum.  The offset is the floor of the largest
// x c2 of the wave's earlier chunks (for its first chunk, of that chunk's
// own maximum); a chunk whose lane sums exceed 2^8 (a logit well above
// that), or hold a NaN or inf, is re-read and redone from its exact
// maximum.  The re-read keeps the first pass's registers free as
// soon as each vector's terms are taken.
template <int DT, bool VEC>
__device__ __forceinline__ SoftChunk soft_chunk(uint4 (&buf)[kLoads], float c2, const char* row, int c0, int c1,
                                                int lane, bool first, SoftAcc& sa, float (&emax)[kLoads]) {
  constexpr int VE = Fmt<DT>::VE;
  SoftChunk out;
  out.ok = true;
  if (first) {
    // the wave's first chunk: its exact maximum (once per wave)
    float r = -kInf;
#pragma unroll
    for (int i = 0; i < kLoads; ++i)
#pragma unroll
      for (int k = 0; k < VE; ++k) r = fmaxf(r, elem<DT>(buf[i], k));
    r = wave_max(r);
    if (r > -kInf) raise_offset(sa, r * c2);
    unpack_barrier(buf);  // unpack again below rather than hold 64 values
  }
  float em;
  out.zt = exp_terms<DT>(buf, c2, sa.o, emax, &em);
  if (__ballot(!(out.zt <= 256.0f)) != 0) {
    // rare: re-read the chunk
    load_chunk<DT, VEC>(buf, row, c0, c1, lane);
    bool nf;
    const float mx = chunk_max<DT>(buf, &nf);
    out.zt = 0.0f;
    em = 0.0f;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) emax[i] = 0.0f;
    if (nf) {
      out.ok = false;
      return out;
    }
    if (mx > -kInf) {
      raise_offset(sa, mx * c2);
      out.zt = exp_terms<DT>(buf, c2, sa.o, emax, &em);
      if (__ballot(!(out.zt < kInf)) != 0) {
        out.ok = false;
        return out;
      }
    }
  }
  sa.z += (double)out.zt;
  out.o = sa.o;
  out.em = wave_max_nonneg(em);
  if (out.em > 0.0f) {
    // the chunk maximum x c2, from its largest term; the next chunk's offset
    const float xc2 = __builtin_amdgcn_logf(out.em) + sa.o;
    sa.lt = fmaxf(sa.lt, xc2);
    raise_offset(sa, xc2);
  }
  return out;
}

// ========================================================= selection ====

// Orders the wave's LDS accesses (and keeps the compiler from moving them).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// A work-group barrier that orders LDS accesses only.  __syncthreads also
// waits for every global load the wave has in flight (its release fence
// covers global memory); the row kernel's waves exchange data through LDS
// alone, and keep their loads in flight across its barriers.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
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

struct Hist {  // selection histogram: counts and fixed-point masses per digit
  uint32_t hc[256];
  unsigned long long hm[256];
};

struct SelOut {
  float T;
  bool reached;
  uint32_t n_keep;
  unsigned long long m_keep, m_above;
};

// One digit of a selection: scans the 256 digits from the top down, with
// the counts and masses above them (above_c, above_m), for the first digit
// whose inclusive cumulative count (top-k) or fixed-point mass (nucleus)
// reaches `target`; without one (not reached), the lowest non-empty digit.
// bin(dg, c, m) gives digit dg's count and mass.  Adds the exclusive sums
// at the digit to above_*, and returns the digit with its own count and
// mass in last_*.
template <class Bin>
__device__ __forceinline__ int pick_digit(Bin&& bin, bool by_mass, unsigned long long target,
                                          unsigned long long& above_c, unsigned long long& above_m,
                                          unsigned long long& last_c, unsigned long long& last_m, bool& reached,
                                          int lane) {
  // lane l holds digits 255 - 4l - j, j = 0..3: descending over the wave
  unsigned long long c[4], m[4], lc = 0, lm = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    bin(255 - 4 * lane - j, c[j], m[j]);
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
  above_c += ac;
  above_m += am;
  // the digit's own count and mass, from the lane holding it
  last_c = lane_at(J == 0 ? c[0] : J == 1 ? c[1] : J == 2 ? c[2] : c[3], L);
  last_m = lane_at(J == 0 ? m[0] : J == 1 ? m[1] : J == 2 ? m[2] : m[3], L);
  return 255 - 4 * L - J;
}
// The same over a histogram's counts and masses.
__device__ __forceinline__ int pick_digit_hist(const Hist& ws, bool by_mass, unsigned long long target,
                                          unsigned long long& above_c, unsigned long long& above_m,
                                          unsigned long long& last_c, unsigned long long& last_m, bool& reached,
                                          int lane) {
  return pick_digit(
      [&](int dg, unsigned long long& c, unsigned long long& m) {
        c = ws.hc[dg];
        m = ws.hm[dg];
      },
      by_mass, target, above_c, above_m, last_c, last_m, reached, lane);
}

__device__ __forceinline__ void clear_histogram(Hist& ws, int lane) {
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
__device__ __forceinline__ SelOut wave_select(Each&& each, bool by_mass, unsigned long long target, Hist& ws,
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
    const int dg = pick_digit_hist(ws, by_mass, target, above_c, above_m, last_c, last_m, reached, lane);
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
// selection: every digit is one bf16 value, so the histogram counts
// elements only and each digit's mass is its count times the value's mass
// (mass_of), the same integers as adding the elements' masses one by one.
__device__ __forceinline__ bool narrow_range(float lo, float hi) {
  return lo <= hi && (fkey(hi) >> 16) - (fkey(lo) >> 16) < 256u;
}

// Fixed-point mass of a logit, in units of the row's largest term:
// 2^((x - M) c2) = 2^(x c2 - oM) 2^(oM - M c2), with oM = M c2 in fp32 and
// the second factor (fM) exact in fp64.
__device__ __forceinline__ unsigned long long mass_of(float x, float c2, float oM, double fM) {
  return (unsigned long long)((double)__builtin_amdgcn_exp2f(fmaf(x, c2, -oM)) * fM * kFix + 0.5);
}

// The bf16 value whose 16-bit order key (fkey(x) >> 16) is k16.
__device__ __forceinline__ float bf16_of_key(uint32_t k16) {
  return key_value((k16 << 16) | ((k16 & 0x8000u) ? 0u : 0xFFFFu));
}

template <bool B>
struct BoolTag {
  static constexpr bool value = B;
};

// Template mode of the row kernel for calls with a per-sequence mode array:
// every work-group takes its own row's path, in one launch.
constexpr int kAnyMode = 4;
// What one wave of the row kernel found over its part of the row.
struct WaveRec {
  double z;        // plain / nucleus: the sum of 2^(x c2 - o) over the wave's logits
  float m;         // the largest logit (-inf if none is finite)
  float o;         // the exponent offset of z
  int arg;         // greedy: the lowest index holding m
  uint32_t flags;  // kCfNonFinite
};

constexpr int kDrawTiles = 4;   // tiles of a row draw whose loads are in flight together
constexpr int kTileCap = 384;   // tile sums per wave of a row draw held in LDS
constexpr int kMaxRows = 2 * kMaxK + 1;

template <int NW>
struct SmemSeq {
  RowRec rows[kMaxRows];
  double rd[NW];
  int ri[NW];
  uint32_t misc[4];
  double rx[2];
  int rj[NW];
  // a draw located by precomputed sums: its range, the weight before it,
  // the row's total and its first / last tokens with weight
  int dl_lo, dl_hi, dl_nzlo, dl_nzhi, dl_beyond;
  double dl_base, dl_S;
  double ua[kWave];  // uniforms of the accept tests at positions 0..63, and of
  double ud[kWave];  //   the resample (t < K_b) or bonus (t = K_b) draws
  double tsum[NW][kTileCap];
};

// Stores and loads that are coherent across the chip's L2s (agent scope,
// relaxed): the parts of a split row exchange their records and lists
// through them.  A part's stores are complete (vmcnt(0)) before its
// arrival is counted, and the last part loads only after it has seen every
// arrival, so no fence of a whole L2 is needed (such fences at the end of
// every work-group cost more than the balance gains).
__device__ __forceinline__ void cstore64(void* p, uint64_t v) {
  __hip_atomic_store(static_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t cload64(const void* p) {
  return __hip_atomic_load(static_cast<uint64_t*>(const_cast<void*>(p)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t pack2(uint32_t lo, uint32_t hi) { return (uint64_t)lo | ((uint64_t)hi << 32); }
// Row records, kept entries and chunk sums through coherent stores and
// loads (the sequence step of a fused call reads what other work-groups of
// the same kernel wrote).
static_assert(sizeof(RowRec) == 48 && sizeof(ChunkRec) == 16 && sizeof(KeptEntry) == 8, "record layouts");
template <class T>
__device__ __forceinline__ void cstore_rec(T* p, const T& v) {
  uint64_t w[sizeof(T) / 8];
  __builtin_memcpy(w, &v, sizeof(T));
#pragma unroll
  for (int k = 0; k < (int)(sizeof(T) / 8); ++k) cstore64(reinterpret_cast<uint64_t*>(p) + k, w[k]);
}
template <bool kCoh, class T>
__device__ __forceinline__ T load_rec(const T* p) {
  if constexpr (!kCoh) {
    return *p;
  } else {
    uint64_t w[sizeof(T) / 8];
#pragma unroll
    for (int k = 0; k < (int)(sizeof(T) / 8); ++k) w[k] = cload64(reinterpret_cast<const uint64_t*>(p) + k);
    T v;
    __builtin_memcpy(&v, w, sizeof(T));
    return v;
  }
}

struct RowSmem {
  uint4 cv[kRowWaves][kCandVecs];  // candidate vectors of each wave, in vocabulary order
  int ci[kRowWaves][kCandVecs];    // the vocabulary index of each one's first logit
  float ck[kRowWaves][kCandVecs];  // while listing: the largest logit of each vector (within 2^-8 / c2)
  WaveRec wrec[kRowWaves];         // each wave's record
  Hist h[3];                       // the finish's selection histograms (rotating)
  float pub[kRowWaves];            // each wave's running maximum (nucleus) or cut (top-k)
  float ucut[kRowWaves];           // the largest listing cut each wave used
  int ncand[kRowWaves];            // candidates listed by each wave, -1 after an overflow
  int wsum[kRowWaves];             //   each wave's part of a work-group sum
  unsigned long long msum[kRowWaves];  //   each wave's part of a kept mass
  int pseg[kMaxParts * kRowWaves + 1];  // split rows: where each part-wave's list starts in the merged order
  int parrive;                     //   the part's arrival number
  int pinc;                        //   a part's list overflowed
  float pg, pu;                    //   the parts' largest maximum / cut, and listing cut
  int pwin[8][kRowWaves];          //   candidates per listing window, per wave
};

// A row work-group's LDS: the row's streaming and finish, then, in a fused
// call, the sequence step of the sequence's last row (4 waves).
union RowSeqSmem {
  RowSmem r;
  SmemSeq<kRowWaves> q;
};
static_assert(offsetof(RowSmem, parrive) >= sizeof(SmemSeq<kRowWaves>),
              "the arrival number is read after the sequence step may write its LDS");

template <int DT, bool VEC, int NW, bool kCoh>
__device__ __forceinline__ void seq_body(const KParams& P, int b, const SeqParams& sp, SmemSeq<NW>& sm);
__device__ __forceinline__ void write_error(const KParams& P, int b, uint32_t st, int first, int stride);

__device__ __forceinline__ float lds_load_relaxed(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_store_relaxed(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// The largest value the row's waves have published so far.
__device__ __forceinline__ float published_max(const RowSmem& sm) {
  float g = -kInf;
#pragma unroll
  for (int w = 0; w < kRowWaves; ++w) g = fmaxf(g, lds_load_relaxed(&sm.pub[w]));
  return g;
}

// Lists the lane's vectors flagged in `mask` (slot i holds logits
// c0 + (i * 64 + lane) * VE + [0, VE), its data in buf[i]) in the wave's
// LDS list from position n, as (data, first vocabulary index, key), in
// (slot, lane) order, which is increasing vocabulary index.  Returns the new
// count; entries beyond kCandVecs are counted, not stored.
// key(i) gives slot i's key; it is evaluated only for flagged slots.
template <class Key>
__device__ __forceinline__ int list_vectors(RowSmem& sm, int wv, int n, uint32_t mask, Key&& key,
                                            const uint4 (&buf)[kLoads], int c0, int ve, int lane) {
  const int e0 = c0 + lane * ve;
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const bool h = (mask >> i) & 1u;
    const uint64_t bal = __ballot(h);
    if (bal) {  // slots with no flagged vector cost one ballot
      if (h) {
        const int pos = n + lanes_below(bal);
        if (pos < kCandVecs) {
          sm.cv[wv][pos] = buf[i];
          sm.ci[wv][pos] = e0 + i * kWave * ve;
          sm.ck[wv][pos] = key(i);
        }
      }
      n += __popcll(bal);
    }
  }
  return n;
}

// Keeps the first n listed vectors of the wave whose key reaches `cut`, in
// order (in place: positions only move down); returns how many.
__device__ __forceinline__ int compact_listed(RowSmem& sm, int wv, int n, float cut, int lane) {
  int m = 0;
  for (int j0 = 0; j0 < n; j0 += kWave) {
    const int j = j0 + lane;
    const bool keep = j < n && sm.ck[wv][j] >= cut;
    const int idx = j < n ? sm.ci[wv][j] : 0;
    const float key = j < n ? sm.ck[wv][j] : 0.0f;
    const uint4 v = j < n ? sm.cv[wv][j] : make_uint4(0, 0, 0, 0);
    const uint64_t bal = __ballot(keep);
    wave_sync();
    if (keep) {
      const int pos = m + lanes_below(bal);
      sm.ci[wv][pos] = idx;
      sm.ck[wv][pos] = key;
      sm.cv[wv][pos] = v;
    }
    m += __popcll(bal);
    wave_sync();
  }
  return m;
}

// Number of the wave's first n listed vectors whose key reaches t.
__device__ __forceinline__ int count_listed(const RowSmem& sm, int wv, int n, float t, int lane) {
  int m = 0;
  for (int j0 = 0; j0 < n; j0 += kWave) m += __popcll(__ballot(j0 + lane < n && sm.ck[wv][j0 + lane] >= t));
  return m;
}

// Top-k: a cut t >= cut such that at least `need` of the wave's first n
// listed vectors have a key (their largest logit) >= t, and as few more as
// the search finds: k vectors each holding a logit >= t make t a lower
// bound of the row's k-th largest logit.  Bisection between cut and the
// largest key; returns cut when no higher value keeps `need` of them.
__device__ __forceinline__ float raise_cut(const RowSmem& sm, int wv, int n, float cut, int need, int lane) {
  float top = -kInf;
  for (int j = lane; j < n; j += kWave) top = fmaxf(top, sm.ck[wv][j]);
  top = wave_max(top);
  float lo = cut, hi = top;  // count(lo) >= need is not known: lo is kept only if it is the best found
  float best = cut;
  if (!(hi > lo)) return cut;
  if (count_listed(sm, wv, n, hi, lane) >= need) return hi;
  for (int it = 0; it < 30; ++it) {
    const float mid = 0.5f * (lo + hi);
    if (!(mid > lo && mid < hi)) break;
    const int m = count_listed(sm, wv, n, mid, lane);
    if (m >= need) {
      best = mid;
      lo = mid;
      if (m <= 2 * need) break;
    } else {
      hi = mid;
    }
  }
  return best;
}

// ---- the finish's selection, over the whole work-group ----
//
// The selection of wave_select over elements known to lie in [lo, hi],
// with the histogram filled by all kThreads threads and every wave picking
// each digit itself from it (the same reads give the same digit), so a
// level costs one barrier.  Three histograms rotate: a level counts into
// sm.h[hb], clears the one after it for the next level, and the one after
// that is still being read by slower waves' previous picks.  hb: in, a
// histogram known to be clear; out, the next such one.
//   bf16 elements spanning fewer than 256 values (narrow_range) take one
// level whose digits are the values themselves: the histogram counts them,
// and each digit's mass is its count times the value's mass.  Otherwise
// MSB-first 8-bit digits; for fp32 only the bits below the prefix shared
// by fkey(lo) and fkey(hi) (fixed top digits would put nearly every
// candidate in one or two bins, whose atomics then serialise).  A nucleus
// selection adds masses per digit; a top-k one counts elements only, and
// its kept mass (keep_mass) is summed once T is known: the same integers.
// each(f, with_mass) calls f(x, mass) for this thread's share of the
// elements (mass only when with_mass is set).
template <int DT, class Each>
__device__ __forceinline__ SelOut wg_select(Each&& each, bool by_mass, unsigned long long target, RowSmem& sm,
                                            int tid, int wv, int lane, float lo, float hi, float c2, float oM,
                                            double fM, int& hb, bool keep_mass = true) {
  static_assert(kThreads == 256, "one histogram bin per thread");
  unsigned long long above_c = 0, above_m = 0, last_c = 0, last_m = 0;
  bool reached = true;
  SelOut r;
  if (DT == SV_BF16 && narrow_range(lo, hi)) {
    const uint32_t kb = (fkey(hi) >> 16) - 255u;  // the key of digit 0
    Hist& h = sm.h[hb];
    each([&](float x, unsigned long long) { atomicAdd(&h.hc[min(255u, (fkey(x) >> 16) - kb)], 1u); }, false);
    const int nx = hb == 2 ? 0 : hb + 1;
    sm.h[nx].hc[tid] = 0;
    sm.h[nx].hm[tid] = 0;
    lds_barrier();
    const int dg = pick_digit(
        [&](int d, unsigned long long& c, unsigned long long& m) {
          const uint32_t n = h.hc[d];
          c = n;
          m = n ? (unsigned long long)n * mass_of(bf16_of_key(kb + (uint32_t)d), c2, oM, fM) : 0ull;
        },
        by_mass, target, above_c, above_m, last_c, last_m, reached, lane);
    hb = nx;
    uint32_t pkey = (kb + (uint32_t)dg) << 16;
    pkey |= (pkey >> 31) ? 0u : 0xFFFFu;
    r.T = key_value(pkey);
    r.reached = reached;
    r.n_keep = (uint32_t)(above_c + last_c);
    r.m_keep = above_m + last_m;
    r.m_above = above_m;
    return r;
  }
  int levels = 2, shift0 = 24;
  uint32_t pkey = 0, pmask = 0;
  if constexpr (DT != SV_BF16) {
    const uint32_t klo = fkey(lo), khi = fkey(hi);
    const uint32_t diff = klo <= khi ? klo ^ khi : 0xFFFFFFFFu;
    const int nb = diff ? 32 - __clz(diff) : 0;  // the varying low bits
    pmask = nb >= 32 ? 0u : ~((1u << nb) - 1u);
    pkey = klo & pmask;
    shift0 = max(nb - 8, 0);
    levels = (shift0 + 7) / 8 + 1;
  }
  for (int lv = 0; lv < levels; ++lv) {
    const int shift = max(shift0 - 8 * lv, 0);
    Hist& h = sm.h[hb];
    each(
        [&](float x, unsigned long long m) {
          const uint32_t key = fkey(x);
          if ((key & pmask) == pkey) {
            const uint32_t dg = (key >> shift) & 255u;
            atomicAdd(&h.hc[dg], 1u);
            if (by_mass) atomicAdd(&h.hm[dg], m);
          }
        },
        by_mass);
    const int nx = hb == 2 ? 0 : hb + 1;
    sm.h[nx].hc[tid] = 0;
    sm.h[nx].hm[tid] = 0;
    lds_barrier();
    const int dg = pick_digit(
        [&](int d, unsigned long long& c, unsigned long long& m) {
          c = h.hc[d];
          m = by_mass ? h.hm[d] : 0ull;
        },
        by_mass, target, above_c, above_m, last_c, last_m, reached, lane);
    hb = nx;
    pkey |= (uint32_t)dg << shift;
    pmask |= 255u << shift;
  }
  if (DT == SV_BF16) pkey |= (pkey >> 31) ? 0u : 0xFFFFu;
  r.T = key_value(pkey);
  r.reached = reached;
  r.n_keep = (uint32_t)(above_c + last_c);
  r.m_keep = above_m + last_m;
  r.m_above = above_m;
  if (!by_mass && keep_mass) {
    // the elements >= T are those counted in n_keep
    const float T = r.T;
    unsigned long long acc = 0;
    each([&](float x, unsigned long long m) { acc += x >= T ? m : 0ull; }, true);
    acc = lane63(wave_scan(acc, 0ull, [](unsigned long long a, unsigned long long b) { return a + b; }));
    if (lane == 0) sm.msum[wv] = acc;
    lds_barrier();
    unsigned long long mk = 0;
#pragma unroll
    for (int w = 0; w < kRowWaves; ++w) mk += sm.msum[w];
    r.m_keep = mk;
    // (msum is written again only after this call's next barrier)
  }
  return r;
}

// The last part of a split row to arrive (its part records from q0 on):
// the parts' wave records are merged into one record (M the largest
// maximum, Z the exact power-of-two rescaling of every sum to the largest
// offset, flags or-ed, the greedy argmax the lowest index holding M) in
// wrec[0], the other three left empty; their candidate lists are read in
// part and wave order, which is vocabulary order, and those at or above the
// row's cut are placed in the work-group's lists as one list of up to
// kRowWaves * kCandVecs vectors (wave w's buffer holding positions 256 w
// on).  A nucleus whose candidates within 10 log2 units of M do not fit
// takes the widest narrower window that fits, as the waves do while
// listing; lists that still do not fit, or a part's overflowed list, leave
// the row to the whole-row selection.  Ends with the records, counts and
// cuts in LDS as the finish reads them (without the barrier).
template <int DT>
__device__ __forceinline__ void merge_parts(const KParams& P, RowSmem& sm, size_t q0, int NP, bool is_topk,
                                            bool is_topp, double ic2, int lane, int wv) {
  constexpr int kSeg = kMaxParts * kRowWaves;
  const int tid = (int)threadIdx.x;
  const int NR = NP * kRowWaves;
  if (wv == 0) {
    double z = 0.0;
    float m = -kInf, o = 0.0f, uc = -kInf, pb = -kInf;
    int arg = 0x7fffffff, ncd = 0;
    uint32_t flags = 0;
    if (lane < NR) {
      const uint64_t* d = reinterpret_cast<const uint64_t*>(&P.phdr[q0 + lane / kRowWaves].w[lane % kRowWaves]);
      const uint64_t w0 = cload64(d), w1 = cload64(d + 1), w2 = cload64(d + 2), w3 = cload64(d + 3),
                     w4 = cload64(d + 4);
      z = __longlong_as_double((long long)w0);
      m = __uint_as_float((uint32_t)w1);
      o = __uint_as_float((uint32_t)(w1 >> 32));
      arg = (int)(uint32_t)w2;
      flags = (uint32_t)(w2 >> 32);
      ncd = (int)(uint32_t)w3;
      uc = __uint_as_float((uint32_t)(w3 >> 32));
      pb = __uint_as_float((uint32_t)w4);
    }
    const bool fin = m > -kInf;  // (a wave with no finite logit has z = 0)
    const float M = wave_max(m);
    const float om = wave_max(fin ? o : -kInf);
    const double zs = wave_sum(fin ? ldexp(z, (int)fmax((double)o - (double)om, -2000.0)) : 0.0);
    const uint32_t fl = wave_or_u(flags);
    const int ag = wave_min_i(fin && m == M ? arg : 0x7fffffff);
    const bool inc = __ballot(lane < NR && ncd < 0) != 0;
    const float ucm = wave_max(uc), gm = wave_max(pb);
    const int cnt = (lane < NR && ncd > 0) ? ncd : 0;
    const int incl = wave_incl_scan_i(cnt, lane);
    if (lane < NR) sm.pseg[lane + 1] = incl;
    if (lane == 0) {
      sm.pseg[0] = 0;
      WaveRec mr;
      mr.z = zs;
      mr.m = M;
      mr.o = M > -kInf ? om : 0.0f;
      mr.arg = ag;
      mr.flags = fl;
      sm.wrec[0] = mr;
      WaveRec e;
      e.z = 0.0;
      e.m = -kInf;
      e.o = 0.0f;
      e.arg = 0x7fffffff;
      e.flags = 0u;
      sm.wrec[1] = e;
      sm.wrec[2] = e;
      sm.wrec[3] = e;
      sm.pg = gm;
      sm.pu = ucm;
      sm.pinc = inc ? 1 : 0;
    }
  }
  lds_barrier();
  const bool lists = is_topk || is_topp;
  bool incomplete = sm.pinc != 0;
  const float g = sm.pg;
  float C = sm.pu;
  int Nk = 0;
  if (lists && !incomplete) {
    const int T = sm.pseg[NR];
    // thread tid reads list positions [j0, j1) of the parts' lists in order
    const int per = (T + kThreads - 1) / kThreads;
    const int j0 = min(T, tid * per), j1 = min(T, j0 + per);
    float key[kSeg];
    int idx[kSeg], pos[kSeg];
    int sg = 0;
#pragma unroll
    for (int k = 0; k < kSeg; ++k) {
      const int j = j0 + k;
      key[k] = -kInf;
      idx[k] = 0;
      pos[k] = -1;
      if (j < j1) {
        while (j >= sm.pseg[sg + 1]) ++sg;
        pos[k] = (int)((q0 * kRowWaves + sg) * kCandVecs) + (j - sm.pseg[sg]);
        const uint64_t w = cload64(&P.pik[pos[k]]);
        idx[k] = (int)(uint32_t)w;
        key[k] = __uint_as_float((uint32_t)(w >> 32));
      }
    }
    // the cut: top-k's largest cut; a nucleus's widest window that fits
    // (10, 8, 6, 5, 4, 3, 2 log2 units below the largest chunk maximum;
    // keys are within 2^-8 / c2 of their vectors' maxima)
    constexpr int kWin = 7;
    float kc[kWin];
#pragma unroll
    for (int wi = 0; wi < kWin; ++wi) {
      const double w = wi == 0 ? (double)kCandLog2 : wi == 1 ? 8.0 : (double)(8 - wi);
      kc[wi] = is_topk ? g : (float)((double)g - w * ic2 - 0.00390625 * ic2);
    }
#pragma unroll
    for (int wi = 0; wi < kWin; ++wi) {
      int c = 0;
#pragma unroll
      for (int k = 0; k < kSeg; ++k) c += (pos[k] >= 0 && key[k] >= kc[wi]) ? 1 : 0;
      c = wave_sum_i(c);
      if (lane == 0) sm.pwin[wi][wv] = c;
    }
    lds_barrier();
    int wsel = -1;
#pragma unroll
    for (int wi = kWin - 1; wi >= 0; --wi) {
      int tot = 0;
#pragma unroll
      for (int w = 0; w < kRowWaves; ++w) tot += sm.pwin[wi][w];
      if (tot <= kRowWaves * kCandVecs && (wi == 0 || !is_topk)) wsel = wi;
    }
    if (wsel < 0) {
      incomplete = true;
    } else {
      const double wsw = wsel == 0 ? (double)kCandLog2 : wsel == 1 ? 8.0 : (double)(8 - wsel);
      float kcs = kc[0];
#pragma unroll
      for (int wi = 1; wi < kWin; ++wi) kcs = wi == wsel ? kc[wi] : kcs;
      C = fmaxf(C, is_topk ? g : (float)((double)g - wsw * ic2));
      int cnt = 0;
#pragma unroll
      for (int k = 0; k < kSeg; ++k) cnt += (pos[k] >= 0 && key[k] >= kcs) ? 1 : 0;
      const int incl = wave_incl_scan_i(cnt, lane);
      if (lane == kWave - 1) sm.wsum[wv] = incl;
      lds_barrier();
      int off = incl - cnt;
#pragma unroll
      for (int w = 0; w < kRowWaves; ++w) {
        const int sw = sm.wsum[w];
        off += w < wv ? sw : 0;
        Nk += sw;
      }
      // the vectors of the positions kept, placed in order
#pragma unroll
      for (int k = 0; k < kSeg; ++k) {
        if (pos[k] >= 0 && key[k] >= kcs) {
          const uint64_t* dv = reinterpret_cast<const uint64_t*>(P.pvec + pos[k]);
          const uint64_t a = cload64(dv), bb = cload64(dv + 1);
          sm.cv[off / kCandVecs][off % kCandVecs] = make_uint4((uint32_t)a, (uint32_t)(a >> 32), (uint32_t)bb,
                                                               (uint32_t)(bb >> 32));
          sm.ci[off / kCandVecs][off % kCandVecs] = idx[k];
          sm.ck[off / kCandVecs][off % kCandVecs] = key[k];
          ++off;
        }
      }
    }
  }
  if (tid < kRowWaves) {
    sm.ncand[tid] = (lists && incomplete) ? (tid == 0 ? -1 : 0) : min(max(Nk - kCandVecs * tid, 0), kCandVecs);
    sm.ucut[tid] = C;
  }
}

// FUSE: the launch runs the sequence step too (one filter only); its own
// instance, so that launches without it keep the plain kernel's registers.
template <int DT, bool VEC, int MODE, bool FUSE>
__global__ __launch_bounds__(kThreads, 3) void row_kernel(const KParams P) {
  constexpr int VE = Fmt<DT>::VE;
  constexpr bool kAny = MODE == kAnyMode;
  static_assert(!(FUSE && kAny), "a call with a mode per sequence is not fused");
  // (the sequence step of a fused call reuses the finished row's LDS)
  __shared__ RowSeqSmem U;
  RowSmem& sm = U.r;
  const int lane = (int)__lane_id();
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  const int R = P.R, S = P.S;
  // work-group blockIdx.x streams the launch's row rowg whole, or part
  // `part` of NP of it (rows from P.full on).  The parts come first: the
  // wave scheduler favours older waves, and a split row's parts must end
  // early for its hand-off to be hidden.
  const uint32_t bid = blockIdx.x;
  const bool split = bid < (uint32_t)P.nsplit;
  const int NP = split ? P.parts : 1;
  const uint32_t rowg = split ? (uint32_t)P.full + bid / (uint32_t)NP : bid - (uint32_t)P.nsplit;
  const int part = split ? (int)(bid % (uint32_t)NP) : 0;
  // rows launched per sequence: all 2 K_max + 1, or the K_max + 1 target
  // rows of a greedy call without the draft's logits
  const int Rl = P.draft ? R : P.K_max + 1;
  const int b = P.b_base + (int)(rowg / (uint32_t)Rl);
  const int r = (int)(rowg % (uint32_t)Rl);
  // Row r of the padded layout: target positions 0..K_max, then draft
  // positions; whether the sequence uses it depends on its K_b.
  // Whole work-groups return here, before any barrier.
  const bool tgt = r <= P.K_max;
  const int t = tgt ? r : r - P.K_max - 1;
  if (!tgt && P.draft == nullptr) return;  // greedy calls without draft logits
  const char* row = static_cast<const char*>(row_ptr<DT>(P, b, tgt, t));
  // the work-group streams chunks [ps, pe) of the row, wave wv chunks [cb, ce)
  const int PS = (S + NP - 1) / NP;
  const int ps = min(S, part * PS), pe = min(S, ps + PS);
  const int per = (pe - ps + kRowWaves - 1) / kRowWaves;
  const int cb = min(pe, ps + wv * per), ce = min(pe, cb + per);
  constexpr int ES = Fmt<DT>::ES;
  const int row_bytes = P.V * ES;
  // The sequence's parameters come through the scalar cache, so that using
  // them never waits for a chunk of logits in flight (under a full stream
  // a vector load can take microseconds).  The first chunk's loads go out
  // once K_b is known (padding rows are never read: theirs read nothing,
  // past the row's end), before the other parameters are used.
  uint4 A[kLoads], B[kLoads];
  const __amdgpu_buffer_rsrc_t rs = row_resource(row, row_bytes);
  auto off = [&](int cc) { return cc < ce ? cc * P.L * ES : row_bytes; };
  // (a per-sequence mode is one byte, loaded by the vector unit before the
  // chunk, so that its wait does not include the chunk's)
  const SeqParams raw = raw_params<!kAny>(P, b, raw_mode(P, b));
  const bool used = tgt ? t <= raw.Kb : t < raw.Kb;
  if constexpr (VEC) issue_chunk<DT>(A, rs, used ? off(cb) : row_bytes, lane);
  const SeqParams sp = check_params(P, raw);
  if (!sp.valid) {
    // the sequence step reports the parameter error: in a fused call the
    // work-group of the sequence's first row (or its first part)
    if (FUSE && r == 0 && part == 0) write_error(P, b, SV_ST_PARAM, (int)threadIdx.x, kThreads);
    return;
  }
  if (!used) return;      // a padding row
  // the row's filter (work-group uniform)
  // (a greedy instance only ever sees greedy rows: the mode is never remapped)
  const bool is_greedy = MODE == SV_GREEDY || (kAny && sp.mode == SV_GREEDY);
  const bool is_topk = (MODE == SV_TOPK || kAny) && sp.mode == SV_TOPK;
  const bool is_topp = (MODE == SV_TOPP || kAny) && sp.mode == SV_TOPP;
  const bool is_plain = !is_greedy && !is_topk && !is_topp;
  const size_t rid = (size_t)b * R + r;
  const size_t slot0 = rid * S;
  const float c2 = (float)sp.c2;
  // The row's draft token: a vector load issued here and first used after
  // the stream, which also loads the token's logit.  (Through the scalar
  // cache its wait would share the LDS counter, and the barrier below would
  // hold the stream until the token arrived, behind every row's first chunk;
  // a load of the logit here would do the same.)
  int tok = INT32_MIN;
  if (t < sp.Kb) {
    const __amdgpu_buffer_rsrc_t trs = row_resource(reinterpret_cast<const char*>(P.tokens + (size_t)b * P.K_max),
                                                    P.K_max * 4);
    // (an offset the compiler cannot see is uniform keeps the value in a
    // vector register, so that nothing waits for it before it is used)
    int z = 0;
    asm volatile("" : "+v"(z));
    tok = (int)__builtin_amdgcn_raw_buffer_load_b32(trs, t * 4 + z, 0, 0);
  }
  if (lane == 0) lds_store_relaxed(&sm.pub[wv], -kInf);
  if (P.prio) __builtin_amdgcn_s_setprio(3);
  lds_barrier();

  // ---- streaming: wave wv takes chunks [cb, ce) ----
  // Each lane accumulates over all of the wave's chunks on its own (softmax
  // sums, maxima, the greedy candidate); the wave reduces once, after its
  // last chunk.  Only the top-k and nucleus candidate lists, and the chunk
  // sums of plain target rows, are built chunk by chunk.
  int nc = 0;            // candidate vectors listed by this wave
  bool over = false;     // the wave's candidate buffer overflowed
  float run = -kInf;     // this wave's running maximum (nucleus) or cut (top-k)
  float ucut = -kInf;    // the largest listing cut this wave used
  const double ic2 = uniform_d(1.0 / (double)c2);
  const float ic2f = (float)ic2;
  const bool chunk_sums = is_plain && tgt;  // the bonus draw of a plain row locates its chunk
  bool bad = false;      // wave-uniform: a NaN or +inf was seen
  SoftAcc sa;            // plain / nucleus
  sa.z = 0.0;
  sa.o = -kInf;
  sa.lt = -kInf;
  float lmax = -kInf;    // greedy: the lane's largest logit; top-k: the wave's
  int lvec = -1;         // greedy: first index of the lane's first vector holding lmax
  // Reduces chunk c, held in buf (its tail masked first when the row ends
  // inside it and `mask` is set).
  auto do_chunk = [&](const int c, uint4 (&buf)[kLoads], bool mask) {
    const int c0 = c * P.L, c1 = min(P.V, c0 + P.L);
    const int ln = fresh_lane(lane);
    // Every path waits for this chunk's loads here, and only for them: a
    // path that left them in flight (a wave that stops early) would make
    // the loop's next iteration wait for all loads, the next chunk's too.
    unpack_barrier(buf);
    if (mask && c1 - c0 < P.L) mask_chunk<DT>(buf, c0, c1, ln);
    if (bad) return;
    if (is_greedy) {
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
        // strictly larger: the lane's earlier vector (lower index) keeps ties
        if (m > lmax) {
          lmax = m;
          lvec = c0 + (i * kWave + ln) * VE;
        }
      }
      bad = __ballot(nf) != 0;
    } else if (is_topk) {
      float vmax[kLoads];
      bool nf;
      const float mx = vector_maxima<DT>(buf, vmax, &nf);
      if (nf) {
        bad = true;
        return;
      }
      lmax = fmaxf(lmax, mx);
      if (over) return;
      // Every cut published so far is a lower bound of the row's k-th
      // largest logit (some chunk holds k vectors at or above it); this
      // chunk may raise it with its own.
      float cut = fmaxf(run, published_max(sm));
      const int need = sp.topk;
      const int capk = min(kCandVecs, max(2 * need, 64));
      // a chunk with many vectors above the cut raises it with its own
      if (mx > cut && need <= kCandVecs && count_vectors_ge(vmax, cut) > capk) {
        const float kc = choose_cut(vmax, mx, 2.0f, need, capk);
        if (kc < kInf) cut = fmaxf(cut, kc);
      }
      run = cut;
      if (lane == 0) lds_store_relaxed(&sm.pub[wv], run);
      const float cf = fmaxf(cut, -kMaxFinite);  // -inf logits are never candidates
      uint32_t mask = 0;
#pragma unroll
      for (int i = 0; i < kLoads; ++i) mask |= vmax[i] >= cf ? (1u << i) : 0u;
      int n = list_vectors(sm, wv, nc, mask, [&](int i) { return vmax[i]; }, buf, c0, VE, ln);
      if (n > kCandVecs) {
        // Raise the cut to the need-th largest listed key (or near it),
        // drop the entries below it, and list the chunk again.
        wave_sync();
        cut = raise_cut(sm, wv, nc, cut, need, ln);
        nc = compact_listed(sm, wv, nc, cut, ln);
        run = cut;
        if (lane == 0) lds_store_relaxed(&sm.pub[wv], run);
        const float cf2 = fmaxf(cut, -kMaxFinite);
        mask = 0;
#pragma unroll
        for (int i = 0; i < kLoads; ++i) mask |= vmax[i] >= cf2 ? (1u << i) : 0u;
        n = list_vectors(sm, wv, nc, mask, [&](int i) { return vmax[i]; }, buf, c0, VE, ln);
      }
      if (n > kCandVecs) over = true;
      else nc = n;
      ucut = fmaxf(ucut, cut);
    } else {
      float emax[kLoads];
      const SoftChunk ch = soft_chunk<DT, VEC>(buf, c2, row, c0, c1, ln, c == cb, sa, emax);
      if (!ch.ok) {
        bad = true;
        return;
      }
      if (chunk_sums) {
        const double zc = wave_sum((double)ch.zt);
        if (lane == 0) {
          ChunkRec cr;
          cr.z = zc;
          cr.o = ch.o;
          cr.pad = 0;
          if (FUSE) cstore_rec(P.chunks + slot0 + c, cr);
          else P.chunks[slot0 + c] = cr;
        }
      }
      if (is_topp && !over) {
        // the chunk maximum, from its largest term
        const double ma = ch.em > 0.0f ? ((double)__builtin_amdgcn_logf(ch.em) + (double)ch.o) * ic2 : -1e300;
        // List every vector holding a logit >= g - w/c2, g the largest chunk
        // maximum known, with the window w = 10 log2 units first.  A list
        // that would overflow the buffer is first compacted against the
        // window about to be tried, then the chunk is listed again with it,
        // narrowing to 8, 6, 5, 4, 3, 2: everything at or above the
        // narrowest cut used stays listed.
        const double g = fmax(fmax((double)run, ma), (double)published_max(sm));
        float cut = kInf;
        const float o = ch.o;
        auto list_window = [&](double w) {
          cut = (float)(g - w * ic2);
          // x >= cut implies a term >= 2^(cut c2 - o) up to roundings far below the margin
          // (the exponent is >= -10.01: o never exceeds g c2)
          const float thr = __builtin_amdgcn_exp2f((float)((double)cut * (double)c2 - (double)o) - 0.00390625f);
          uint32_t mask = 0;
#pragma unroll
          for (int i = 0; i < kLoads; ++i) mask |= emax[i] >= thr ? (1u << i) : 0u;
          // the key: the vector's largest logit, from its largest term (fp32
          // suffices), taken only for the vectors listed
          return list_vectors(
              sm, wv, nc, mask, [&](int i) { return (__builtin_amdgcn_logf(emax[i]) + o) * ic2f; }, buf, c0, VE, ln);
        };
        int n = list_window(kCandLog2);
        bool done = n <= kCandVecs;
        for (int attempt = 1; attempt < 8 && !done; ++attempt) {
          const double w = attempt == 1 ? kCandLog2 : attempt == 2 ? 8.0 : (double)(9 - attempt);
          // (keys are within 2^-8 / c2 of their vectors' maxima)
          nc = compact_listed(sm, wv, nc, (float)(g - w * ic2 - 0.00390625 * ic2), ln);
          n = list_window(w);
          done = n <= kCandVecs;
        }
        if (done) nc = n;
        if (!done) over = true;
        ucut = fmaxf(ucut, cut);
        run = fmaxf(run, (float)ma);
        if (lane == 0) lds_store_relaxed(&sm.pub[wv], run);
      }
    }
  };
  if constexpr (VEC) {
    // Two chunk buffers: the loads of chunk c + 1 are in flight while chunk
    // c is reduced, so that every wave keeps memory busy.
    // The next chunk's loads are issued whether or not it exists (then at
    // the row's end, where they read nothing), so that the number of loads
    // in flight is always the same and each wait is for one chunk only.
    // Pairs of chunks: every iteration enters with A(c) in flight and
    // leaves with A(c + 2) in flight, so the loop has no exit in its middle
    // and every path into its head holds the same loads.
    const int n = ce - cb;
    int c = cb;
    for (int k = 0; k + 1 < n; k += 2, c += 2) {
      issue_chunk<DT>(B, rs, off(c + 1), lane);
      do_chunk(c, A, true);
      issue_chunk<DT>(A, rs, off(c + 2), lane);
      do_chunk(c + 1, B, true);
      // In a launch whose work-groups are all resident at once, the wave's
      // issue priority falls as it progresses, so that on a SIMD the waves
      // furthest behind issue first (the arbiter otherwise favours the
      // oldest, and a CU's last row would stream alone at the end).
      if (P.prio) {
        const int pr = 3 - (3 * (k + 2)) / n;
        if (pr >= 3) __builtin_amdgcn_s_setprio(3);
        else if (pr == 2) __builtin_amdgcn_s_setprio(2);
        else if (pr == 1) __builtin_amdgcn_s_setprio(1);
        else __builtin_amdgcn_s_setprio(0);
      }
    }
    if (n & 1) do_chunk(c, A, true);  // the last chunk
    else unpack_barrier(A);           // loads past the row's end
  } else {
    for (int c = cb; c < ce; ++c) {
      uint4 buf[kLoads];
      load_chunk<DT, VEC>(buf, row, c * P.L, min(P.V, c * P.L + P.L), lane);
      do_chunk(c, buf, false);
    }
  }
  // the largest chunk maximum (nucleus) or cut (top-k) known to the work-group
  const float gpub = (is_topk || is_topp) ? fmaxf(run, published_max(sm)) : -kInf;
  if ((is_topk || is_topp) && !over && nc > 0) {
    // Keep the listed vectors that can still hold a kept token: for top-k
    // those at or above the largest cut published, for a nucleus those
    // within 10 log2 units of the largest chunk maximum known (keys are
    // within 2^-8 / c2 of the vectors' maxima).
    const float g = gpub;
    const float fcut = is_topk ? g : (float)((double)g - kCandLog2 * ic2);
    nc = compact_listed(sm, wv, nc, is_topk ? fcut : (float)((double)fcut - 0.00390625 * ic2), lane);
    ucut = fmaxf(ucut, fcut);
  }
  // the draft token's logit, for the finish: its bits, loaded by every lane
  // through the row's resource (an offset past the row reads 0), and
  // decoded only where they are used, so that its load completes under the
  // finish's first steps
  const bool tok_ok = tok != INT32_MIN && tok >= 0 && tok < P.V;
  const int xoff = tok_ok ? tok * ES : row_bytes;
  uint32_t xbits;
  if constexpr (DT == SV_BF16) xbits = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, xoff, 0, 0);
  else xbits = __builtin_amdgcn_raw_buffer_load_b32(rs, xoff, 0, 0);
  {
    // the wave's record
    WaveRec wr;
    wr.z = 0.0;
    wr.m = -kInf;
    wr.o = 0.0f;
    wr.arg = 0x7fffffff;
    wr.flags = bad ? kCfNonFinite : 0u;
    if (!bad) {
      if (is_greedy) {
        // the lowest index of the lane's maximum, in its first vector holding it
        int idx = 0x7fffffff;
        if (lvec >= 0) {
          const uint4 v = load_vec<DT, VEC>(row, lvec, P.V);
#pragma unroll
          for (int k = VE - 1; k >= 0; --k)
            if (elem<DT>(v, k) == lmax) idx = lvec + k;
        }
        wr.m = wave_max(lmax);
        wr.arg = wave_min_i(lmax == wr.m ? idx : 0x7fffffff);
      } else if (is_topk) {
        wr.m = lmax;
      } else {
        wr.m = sa.lt > -kInf ? (float)((double)sa.lt * ic2) : -kInf;
        wr.z = wave_sum(sa.z);
        wr.o = sa.o;
      }
    }
    if (!split) {
      if (lane == 0) {
        sm.wrec[wv] = wr;
        sm.ncand[wv] = over ? -1 : nc;
        sm.ucut[wv] = ucut;
      }
    } else {
      // a part of a split row: the wave's record and list, for the part
      // that finishes the row
      const size_t qw = ((size_t)(rowg - (uint32_t)P.full) * NP + part) * kRowWaves + wv;
      if (lane == 0) {
        uint64_t* d = reinterpret_cast<uint64_t*>(&P.phdr[qw / kRowWaves].w[wv]);
        cstore64(d + 0, (uint64_t)__double_as_longlong(wr.z));
        cstore64(d + 1, pack2(__float_as_uint(wr.m), __float_as_uint(wr.o)));
        cstore64(d + 2, pack2((uint32_t)wr.arg, wr.flags));
        cstore64(d + 3, pack2((uint32_t)(over ? -1 : nc), __float_as_uint(ucut)));
        cstore64(d + 4, pack2(__float_as_uint(gpub), 0u));
      }
      wave_sync();  // the wave's own list writes
      const int nl = over ? 0 : nc;
      for (int j = lane; j < nl; j += kWave) {
        const uint4 v = sm.cv[wv][j];
        uint64_t* dv = reinterpret_cast<uint64_t*>(P.pvec + qw * kCandVecs + j);
        cstore64(dv, pack2(v.x, v.y));
        cstore64(dv + 1, pack2(v.z, v.w));
        cstore64(P.pik + qw * kCandVecs + j, pack2((uint32_t)sm.ci[wv][j], __float_as_uint(sm.ck[wv][j])));
      }
    }
  }
  if (split) {
    // Count this part's arrival once every store of its waves is complete;
    // the last part of the row merges and finishes it, the others end here.
    const uint32_t srow = rowg - (uint32_t)P.full;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();
    if (threadIdx.x == 0)
      sm.parrive = __hip_atomic_fetch_add(&P.pcount[srow], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    lds_barrier();
    if (sm.parrive != NP - 1) return;  // (work-group uniform)
    if (threadIdx.x == 0) __hip_atomic_store(&P.pcount[srow], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    merge_parts<DT>(P, sm, (size_t)srow * NP, NP, is_topk, is_topp, ic2, lane, wv);
  }
  __builtin_amdgcn_s_setprio(0);
  sm.h[0].hc[threadIdx.x] = 0;  // the finish's first selection counts into these
  sm.h[0].hm[threadIdx.x] = 0;
  lds_barrier();

  // ---- finish ----
  {
  // Every wave derives the row's statistics from the wave records; the
  // selection and the kept list of a top-k / nucleus row use the whole
  // work-group, other rows only wave 0.
  const int tid = (int)threadIdx.x;
  RowRec rr;
  rr.M = -kInf;
  rr.T = -kInf;
  rr.c2 = (double)c2;
  rr.Zs = 1.0;
  rr.pid = __builtin_nan("");
  rr.g = -1;
  rr.n_keep = -1;
  rr.flags = 0;
  rr.pad = 0;
  // every record and list count read at once (LDS round trips in a row are
  // the finish's latency)
  WaveRec wrs[kRowWaves];
  int ncw[kRowWaves];
  float ucw[kRowWaves];
#pragma unroll
  for (int w = 0; w < kRowWaves; ++w) {
    wrs[w] = sm.wrec[w];
    ncw[w] = sm.ncand[w];
    ucw[w] = sm.ucut[w];
  }
  float mx = -kInf;
  uint32_t fl = 0;
#pragma unroll
  for (int w = 0; w < kRowWaves; ++w) {
    mx = fmaxf(mx, wrs[w].m);
    fl |= wrs[w].flags;
  }
  const float M = mx;
  rr.M = M;
  if ((fl & kCfNonFinite) || !(M < kInf) || isnan(M)) rr.flags |= SV_ST_NONFINITE;
  else if (M == -kInf) rr.flags |= SV_ST_EMPTY;

  double Z = 0.0;
  if (!(rr.flags & kErrBits) && (is_plain || is_topp)) {
    // Z = sum_w z_w 2^(o_w - M c2): the offsets o_w are integers, so with
    // F = floor(M c2) each 2^(o_w - F) is exact and one fp64 exp2 of
    // F - M c2 (in (-1, 0]; M c2 is exact in fp64) scales the sum.
    const double mc2 = (double)M * (double)c2;
    const double F = floor(mc2);
#pragma unroll
    for (int w = 0; w < kRowWaves; ++w) {
      // (a wave with no finite logit has z = 0 and o = -inf or 0)
      const double zw = ldexp(wrs[w].z, (int)fmax((double)wrs[w].o - F, -2000.0));
      Z += wrs[w].m > -kInf ? zw : 0.0;
    }
    Z *= exp2(F - mc2);
    if (!(Z > 0.0) || !(Z < 1e300)) rr.flags |= SV_ST_NONFINITE;
    else if (chunk_sums) rr.flags |= kRfChunks;
  }
  const bool selecting = !(rr.flags & kErrBits) && (is_topk || is_topp);  // work-group uniform
  if (!selecting && wv != 0) {
    // (in a fused call every wave joins the sequence step)
    if constexpr (FUSE) goto arrive;
    return;
  }

  const float oM = M * c2;
  const double fM = exp2_small((double)oM - (double)M * (double)c2);
  bool list_ok = false;
  // the candidate vectors: the waves' buffers one after another
  int pre[kRowWaves + 1];
  float C = -kInf;  // every token >= C lies in a listed vector (+inf: incomplete)
  pre[0] = 0;
  bool incomplete = false;
#pragma unroll
  for (int w = 0; w < kRowWaves; ++w) {
    incomplete |= ncw[w] < 0;
    C = fmaxf(C, ucw[w]);
    pre[w + 1] = pre[w] + max(ncw[w], 0);
  }
  if (incomplete) C = kInf;
  const int N = pre[kRowWaves];
  auto vec_at = [&](int j, uint4& v, int& e0) {
    const int w = (j >= pre[1]) + (j >= pre[2]) + (j >= pre[3]);
    const int pos = j - (w == 0 ? 0 : w == 1 ? pre[1] : w == 2 ? pre[2] : pre[3]);
    v = sm.cv[w][pos];
    e0 = sm.ci[w][pos];
  };
  if (!(rr.flags & kErrBits)) {
    if (is_plain) {
      rr.Zs = Z;
    } else if (is_greedy) {
      int best = 0x7fffffff;
#pragma unroll
      for (int w = 0; w < kRowWaves; ++w)
        if (wrs[w].m == M) best = min(best, wrs[w].arg);
      rr.g = best;
      rr.T = M;
      rr.n_keep = 1;
    } else {
      const bool by_mass = is_topp;
      unsigned long long target;
      if (by_mass) {
        const double tt = (double)sp.topp * Z * kFix;
        target = tt < 1.0 ? 1ull : (unsigned long long)tt;
      } else {
        target = (unsigned long long)sp.topk;
      }
      // an upper bound of every logit of the row: M comes from the chunks'
      // largest terms, within a few ulps of the largest logit
      const float Mhi = M + (fabsf(M) + 1.0f) * 0.001953125f;
      // Candidates spanning fewer than 256 bf16 values take one histogram
      // pass over all of them.  Otherwise a nucleus first tries the cut 8
      // log2 units below the row maximum (the lists reach 10), then C; a
      // top-k selection runs over every candidate >= C at once.
      const bool narrow = DT == SV_BF16 && C < kInf && narrow_range(fmaxf(C, -kMaxFinite), Mhi);
      int hb = 0;  // a clear histogram (cleared before the finish)
      const float C1 = (by_mass && !narrow) ? fmaxf(C, (float)((double)M - 8.0 / (double)c2)) : C;
      SelOut so;
      bool ok = false;
      for (int pass = 0; pass < 2 && !ok && C < kInf; ++pass) {
        const float Cu = pass == 0 ? C1 : C;
        if (pass == 1 && !(C1 > C)) break;
        const float Cuf = fmaxf(Cu, -kMaxFinite);  // -inf padding never passes
        so = wg_select<DT>(
            [&](auto&& f, bool with_mass) {
              for (int j = tid; j < N; j += kThreads) {
                uint4 v;
                int e0;
                vec_at(j, v, e0);
#pragma unroll
                for (int k = 0; k < VE; ++k) {
                  const float x = elem<DT>(v, k);
                  if (x >= Cuf) f(x, with_mass ? mass_of(x, c2, oM, fM) : 0ull);
                }
              }
            },
            by_mass, target, sm, tid, wv, lane, Cuf, Mhi, c2, oM, fM, hb);
        ok = so.reached && so.T >= Cu;
      }
      if (!ok) {
        // full-row selection by wave 0: re-read the row
        if (wv != 0) {
          if constexpr (FUSE) goto arrive;
          return;
        }
        so = wave_select<DT>(
            [&](auto&& f) {
              for (int e = lane; e < P.V; e += kWave) {
                const float x = load_logit<DT>(row, e);
                f(x, mass_of(x, c2, oM, fM));
              }
            },
            by_mass, target, sm.h[hb], lane);  // (a histogram no wave reads any more)
        rr.flags |= SV_ST_FULLSELECT;
      }
      rr.T = so.T;
      rr.n_keep = (int)so.n_keep;
      rr.Zs = (double)so.m_keep / kFix;
      if (by_mass) {
        const double lo = (double)so.m_above / kFix / Z, hi = (double)so.m_keep / kFix / Z;
        if (fabs(lo - (double)sp.topp) < kWindow || fabs(hi - (double)sp.topp) < kWindow) rr.flags |= SV_ST_MARGIN;
      }
      if (!(rr.Zs > 0.0)) rr.flags |= SV_ST_EMPTY;
      list_ok = ok && tgt && so.n_keep <= (uint32_t)kListMax && !(rr.flags & kErrBits);
    }
  }

  if (list_ok) {
    // the kept set, in vocabulary order: the candidates >= T, compacted in
    // buffer order by the work-group and stored as they are placed
    rr.flags |= kRfListOk;
    KeptEntry* kl = P.kept + ((size_t)b * (P.K_max + 1) + t) * (size_t)min(kListMax, P.V);
    int nk = 0;
    constexpr int kRounds = kRowWaves * kCandVecs / kThreads;
#pragma unroll
    for (int q = 0; q < kRounds; ++q) {
      const int j0 = q * kThreads;
      if (j0 >= N) break;  // work-group uniform
      const int j = j0 + tid;
      const bool have = j < N;
      uint4 v = make_uint4(0, 0, 0, 0);
      int e0 = 0;
      if (have) vec_at(j, v, e0);
      bool pass[VE];
      int cnt = 0;
#pragma unroll
      for (int k = 0; k < VE; ++k) {
        pass[k] = have && elem<DT>(v, k) >= rr.T;
        cnt += pass[k] ? 1 : 0;
      }
      const int incl = wave_incl_scan_i(cnt, lane);
      if (lane == kWave - 1) sm.wsum[wv] = incl;
      lds_barrier();
      int off = nk + incl - cnt, tot = 0;
#pragma unroll
      for (int w = 0; w < kRowWaves; ++w) {
        const int sw = sm.wsum[w];
        off += w < wv ? sw : 0;
        tot += sw;
      }
      // (n_keep <= kListMax, and every kept token is one of these)
#pragma unroll
      for (int k = 0; k < VE; ++k) {
        if (pass[k]) {
          if (off < kListMax) {
            KeptEntry ke;
            ke.idx = e0 + k;
            ke.xq = elem<DT>(v, k);
            if (FUSE) cstore_rec(kl + off, ke);
            else kl[off] = ke;
          }
          ++off;
        }
      }
      nk += tot;
      if (j0 + kThreads < N) lds_barrier();  // the next round writes wsum again
    }
  }

  if (tid == 0) {
    if (tok != INT32_MIN) {  // this row scores a draft token
      if (!tok_ok) {
        rr.flags |= SV_ST_TOKEN;
      } else if (!(rr.flags & kErrBits)) {
        if (is_greedy) rr.pid = tok == rr.g ? 1.0 : 0.0;
        else {
          const float xtok = __uint_as_float(DT == SV_BF16 ? xbits << 16 : xbits);
          rr.pid = xtok >= rr.T ? exp2(((double)xtok - (double)M) * (double)c2) / rr.Zs : 0.0;
        }
      }
    }
    if (FUSE) cstore_rec(P.rows + rid, rr);
    else P.rows[rid] = rr;
  }
  }
arrive:
  if constexpr (FUSE) {
    // A fused call: once every output of this row is complete, count its
    // arrival; the sequence's last row to arrive runs the accept walk and
    // the draw, with 4 waves, on records read back with coherent loads.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();
    const uint32_t sq = (uint32_t)(b - P.b_base);
    if (threadIdx.x == 0)
      sm.parrive = __hip_atomic_fetch_add(&P.scount[sq], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    lds_barrier();
    const int rows_used = sp.Kb + 1 + (P.draft ? sp.Kb : 0);
    if (sm.parrive != rows_used - 1) return;  // (work-group uniform)
    if (threadIdx.x == 0) __hip_atomic_store(&P.scount[sq], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    seq_body<DT, VEC, kRowWaves, true>(P, b, sp, U.q);
  }
}

// ===================================================== sequence kernel ====
//
// One work-group per sequence.  The row records of its 2 K_b + 1 rows come
// from the row kernel; wave 0 runs the accept walk, finds the first
// rejection and draws the resampled or bonus token from the target's kept
// set; a draw that needs the full rows (plain rows, large kept sets) is
// done by the whole work-group.

constexpr int kSeqThreads = kSeqWaves * kWave;  // (the work-group of small batches)

// ------------------------------------------------------------- draws ----

struct Draw {
  int y;
  uint32_t flags;
};

template <int NW>
__device__ __forceinline__ int seq_min_i(int v, SmemSeq<NW>& sm) {
  v = wave_min_i(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sm.ri[threadIdx.x >> 6] = v;
  __syncthreads();
  int s = sm.ri[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) s = min(s, sm.ri[w]);
  return s;
}
template <int NW>
__device__ __forceinline__ int seq_max_i(int v, SmemSeq<NW>& sm) {
  v = wave_max_i(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sm.ri[threadIdx.x >> 6] = v;
  __syncthreads();
  int s = sm.ri[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) s = max(s, sm.ri[w]);
  return s;
}
// Exclusive prefix over the work-group in thread order; *total = the sum.
template <int NW>
__device__ __forceinline__ double seq_exclusive_scan(double v, double* total, SmemSeq<NW>& sm) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const double inc = wave_incl_scan(v, lane);
  __syncthreads();
  if (lane == 63) sm.rd[w] = inc;
  __syncthreads();
  double base = 0.0, tot = 0.0;
#pragma unroll
  for (int j = 0; j < NW; ++j) {
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
// The set comes from the row kernel's kept list kl; a resample reads the
// draft's logits at its tokens from the draft row prow (only the row of the
// first rejection is read, and only there).  The draft's weights are fp32
// terms as in prob().
template <int DT, bool kCoh = false>
__device__ __forceinline__ Draw draw_from_list(const RowRec& rq, bool resample, const RowRec& rp,
                                               const KeptEntry* kl, const void* prow, double u, int lane) {
  constexpr int E = kListMax / kWave;
  const int N = rq.n_keep;  // <= kListMax
  const int ns = (N + kWave - 1) / kWave;
  const RowW wp = row_w(rp);
  double qv[E];
  float pv[E];
  int iv[E];
  const float c2q = (float)rq.c2;
  const float oM = rq.M * c2q;
  const double fM = exp2_small((double)oM - (double)rq.M * (double)c2q);
  const double inv = 1.0 / (rq.Zs * kFix);
  KeptEntry ke[E];
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const int i = j * kWave + lane;
    ke[j].idx = 0;
    ke[j].xq = -kInf;
    if (j < ns && i < N) ke[j] = load_rec<kCoh>(kl + i);
  }
  float xp[E];  // the draft's logits at the kept tokens (a resample only)
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const int i = j * kWave + lane;
    xp[j] = -kInf;
    if (resample && j < ns && i < N) xp[j] = load_logit<DT>(prow, ke[j].idx);
  }
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const int i = j * kWave + lane;
    qv[j] = 0.0;
    pv[j] = 0.0f;
    iv[j] = 0;
    if (j < ns && i < N) {
      iv[j] = ke[j].idx;
      qv[j] = (double)mass_of(ke[j].xq, c2q, oM, fM) * inv;
      if (resample) pv[j] = prob(wp, xp[j]);
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
template <int DT, bool VEC, int NW, bool kCoh = false>
__device__ __forceinline__ Draw draw_from_rows(const KParams& P, const RowRec& rq, bool resample, const RowRec& rp,
                                               const char* qrow, const char* prow, double u, SmemSeq<NW>& sm, int lane,
                                               int wv, const ChunkRec* qrec) {
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
  if (!resample && qrec && (rq.flags & kRfChunks)) {
    // plain bonus draw: the chunk sums give the chunk holding u
    const int S = P.S;
    // kCpt consecutive chunks per thread cover every row (V <= 2^22)
    constexpr int kCpt = (kMaxVocab / (kWave * kLoads * 4) + NW * kWave - 1) / (NW * kWave);
    double wc[kCpt];
    double wsum = 0.0;
#pragma unroll
    for (int j = 0; j < kCpt; ++j) {
      const int c = kCpt * tid + j;
      wc[j] = 0.0;
      if (c < S) {
        const ChunkRec r = load_rec<kCoh>(qrec + c);
        if (r.z > 0.0) wc[j] = r.z * exp2((double)r.o - (double)rq.M * (double)wq.c2) / rq.Zs;
      }
      wsum += wc[j];
    }
    double tot;
    const double ex = seq_exclusive_scan(wsum, &tot, sm);
    int cstar = 0x7fffffff, clast = -1;
    double cb = 0.0;
    double before = ex;
#pragma unroll
    for (int j = 0; j < kCpt; ++j) {
      const int c = kCpt * tid + j;
      if (c < S && wc[j] > 0.0) {
        if (before + wc[j] > u && cstar == 0x7fffffff) {
          cstar = c;
          cb = before;
        }
        clast = c;
      }
      before += wc[j];
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
      d.flags |= SV_ST_LOCATED;
      force_last = cs == 0x7fffffff;  // u beyond the rounded total: the last token of the last chunk
    }
  }
  double* tsum = sm.tsum[wv];  // this wave's tile sums
  double S = 0.0;
  int nzlo = 0x7fffffff, nzhi = -1, per = 0, v0 = 0, v1 = 0;
  for (int pass = 0; pass < 2; ++pass) {
    const int n8 = (hi - lo + 7) / 8;
    per = (n8 + NW - 1) / NW;
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
    for (int w = 0; w < NW; ++w) {
      S += sm.rd[w];
      nzlo = min(nzlo, sm.ri[w]);
    }
    __syncthreads();
    if (lane == 0) sm.ri[wv] = zh;
    __syncthreads();
    nzhi = -1;
#pragma unroll
    for (int w = 0; w < NW; ++w) nzhi = max(nzhi, sm.ri[w]);
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
    for (int w = 0; w < NW; ++w) {
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

// ======================================================= spread draws ====
//
// A residual draw from the rows (n < K_b, plain rows or a kept set not
// listed): inverse CDF over (q_n - p_n)+ in vocabulary order.  Before the
// sequence kernel, one work-group per kDrawSpan tokens of each sequence
// repeats the accept walk (the same uniforms and tests, so the same n) and,
// when the sequence needs such a draw, sums its span's weights; the
// sequence kernel scans the span sums, finds the span holding u * S and
// the token in it.  Both use the weights of weights8 (fp32, in groups of 8
// added pairwise), so the span the sums locate holds the crossing of the
// group-level running sum.

static_assert(kDrawSpan % (8 * kThreads) == 0 && kDrawSpan <= 16 * kSeqThreads,
              "whole groups of 8 per thread in the span kernel; a span within one draw_range of the sequence kernel");

// Loads one word of each 64-byte line of the kernel arguments at once and
// waits for them, so that the scalar cache holds every line before the
// kernel's first parameter tests.  The compiler loads the arguments where
// each test needs them, and a test that branches on a pointer waits for
// its load before the next one issues, so each line's first miss would be
// a round trip of its own.  (In the short, latency-bound kernels only: the
// row kernel's start is hidden behind its first chunk's loads, and there
// the extra wait measured slower.)
__device__ __forceinline__ void warm_kernel_args() {
  typedef __attribute__((address_space(4))) const uint32_t karg_u32;
  static_assert(sizeof(KParams) > 4 * 64 && sizeof(KParams) <= 5 * 64, "the argument block spans five lines");
  karg_u32* ka = (karg_u32*)__builtin_amdgcn_kernarg_segment_ptr();
  const uint32_t w0 = ka[0], w1 = ka[16], w2 = ka[32], w3 = ka[48], w4 = ka[64];
  asm volatile("" ::"s"(w0), "s"(w1), "s"(w2), "s"(w3), "s"(w4));
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void draw_sum_kernel(const KParams P) {
  warm_kernel_args();
  __shared__ double red[kRowWaves];
  __shared__ int rlo[kRowWaves], rhi[kRowWaves];
  __shared__ int sh_n;
  const int D = P.D;
  const int b = P.b_base + (int)(blockIdx.x / (uint32_t)D);
  const int sp_ = (int)(blockIdx.x % (uint32_t)D);
  const int tid = (int)threadIdx.x, lane = (int)__lane_id();
  const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
  const SeqParams sp = load_params(P, b);
  if (!sp.valid || sp.mode == SV_GREEDY) return;  // (whole work-group)
  const int Kb = sp.Kb, KM = P.K_max, R = P.R;
  if (wv == 0) {
    // the walk of the sequence kernel: error rows, then the first t with
    // u_t p_t(d_t) >= q_t(d_t) (K_b <= 64: one lane per position)
    const RowRec* rows = P.rows + (size_t)b * R;
    uint32_t st = 0;
    for (int t = lane; t <= Kb; t += kWave) st |= rows[t].flags;
    for (int t = lane; t < Kb; t += kWave) st |= rows[KM + 1 + t].flags;
    st = wave_or_u(st);
    bool rej = false;
    if (lane < Kb) {
      const uint64_t g = P.row_offset + (uint64_t)b;
      const double ua = uniform24(P.seed, g, (uint32_t)lane, kPurposeAccept);
      rej = !(ua * rows[KM + 1 + lane].pid < rows[lane].pid);
    }
    const uint64_t rb = __ballot(rej);
    const int n = rb ? __ffsll((long long)rb) - 1 : Kb;
    const bool need = !(st & kErrBits) && n < Kb && !(rows[n].flags & kRfListOk);
    if (lane == 0) sh_n = need ? n : -1;
  }
  __syncthreads();
  const int n = sh_n;
  if (n < 0) return;
  const RowRec rq = P.rows[(size_t)b * R + n], rp = P.rows[(size_t)b * R + KM + 1 + n];
  const RowW wq = row_w(rq), wp = row_w(rp);
  const bool all = __builtin_amdgcn_readfirstlane((int)(wq.T == -kInf && wp.T == -kInf)) != 0;
  const char* qrow = static_cast<const char*>(row_ptr<DT>(P, b, true, n));
  const char* prow = static_cast<const char*>(row_ptr<DT>(P, b, false, n));
  const int lo = sp_ * kDrawSpan, hi = min(P.V, lo + kDrawSpan);
  // thread t takes groups t, t + 256, ... of the span (all loads in
  // flight together)
  constexpr int kG = kDrawSpan / 8 / kThreads;
  uint4 aq[kG][2], ap[kG][2];
#pragma unroll
  for (int k = 0; k < kG; ++k) {
    const int e = lo + 8 * (tid + kThreads * k);
    const uint32_t ninf = DT == SV_BF16 ? 0xff80ff80u : 0xff800000u;
    aq[k][0] = aq[k][1] = ap[k][0] = ap[k][1] = make_uint4(ninf, ninf, ninf, ninf);
    if (e < hi) {
      load8<DT, VEC>(P, qrow, e, aq[k]);
      load8<DT, VEC>(P, prow, e, ap[k]);
    }
  }
  double s = 0.0;
  int zl = 0x7fffffff, zh = -1;
#pragma unroll
  for (int k = 0; k < kG; ++k) {
    const int e = lo + 8 * (tid + kThreads * k);
    float w[8];
    const float s8 = weights8<DT>(wq, true, wp, all, aq[k], ap[k], w);
    s += (double)s8;
    if (s8 > 0.0f) {
      zl = min(zl, e);
      zh = max(zh, e + 7);
    }
  }
  s = wave_sum(s);
  zl = wave_min_i(zl);
  zh = wave_max_i(zh);
  if (lane == 0) {
    red[wv] = s;
    rlo[wv] = zl;
    rhi[wv] = zh;
  }
  __syncthreads();
  if (tid == 0) {
    DrawSum ds;
    ds.s = (red[0] + red[1]) + (red[2] + red[3]);
    ds.first = min(min(rlo[0], rlo[1]), min(rlo[2], rlo[3]));
    ds.last = max(max(rhi[0], rhi[1]), max(rhi[2], rhi[3]));
    P.dsums[(size_t)b * D + sp_] = ds;
  }
}

// Inverse CDF over the tokens [lo, hi) of one row (pair) by the whole
// work-group, with two barriers: thread t holds groups 2t and 2t + 1 of 8
// tokens (so at most 16 NW 64 tokens); each wave sums its groups, every
// wave finds from the wave sums the wave whose running sum (from `base`)
// crosses `target` (+inf: none), and that wave finds the group and the
// token in it, the groups' sums and the tokens' weights added as in the
// other draws.  Without a crossing the last token with weight is taken.
struct RangeDraw {
  int y;           // the token, -1 if the range has no weight
  bool crossed;    // the target was crossed (else: the last token with weight)
  int glo, ghi;    // first / last token of the range's groups with weight
  double clo, chi; // running sum just below and at y
  double total;    // the range's weight
};
template <int DT, bool VEC, int NW>
__device__ __forceinline__ RangeDraw draw_range(const KParams& P, const RowW& wq, bool use_p, const RowW& wp,
                                                bool all, const char* qrow, const char* prow, int lo, int hi,
                                                double base, double target, SmemSeq<NW>& sm, int lane, int wv) {
  const int tid = threadIdx.x;
  uint4 aq[2][2], ap[2][2];
  float w[2][8], s8[2];
  int e[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    e[h] = lo + 8 * (2 * tid + h);
    const uint32_t ninf = DT == SV_BF16 ? 0xff80ff80u : 0xff800000u;
    aq[h][0] = aq[h][1] = ap[h][0] = ap[h][1] = make_uint4(ninf, ninf, ninf, ninf);
    if (e[h] < hi) {
      load8<DT, VEC>(P, qrow, e[h], aq[h]);
      if (use_p) load8<DT, VEC>(P, prow, e[h], ap[h]);
    }
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) s8[h] = weights8<DT>(wq, use_p, wp, all, aq[h], ap[h], w[h]);
  const double ts = (double)s8[0] + (double)s8[1];
  const double inc = wave_incl_scan(ts, lane);
  const int fz = wave_min_i(s8[0] > 0.0f ? e[0] : s8[1] > 0.0f ? e[1] : 0x7fffffff);
  const int lz = wave_max_i(s8[1] > 0.0f ? e[1] + 7 : s8[0] > 0.0f ? e[0] + 7 : -1);
  if (lane == kWave - 1) sm.rd[wv] = inc;  // the wave's sum
  if (lane == 0) {
    sm.ri[wv] = fz;
    sm.rj[wv] = lz;
  }
  __syncthreads();
  // the wave whose running sum crosses the target, else the last wave with weight
  double run = base, cb = 0.0, lb = 0.0;
  int cw = -1, lw = -1;
  RangeDraw r;
  r.glo = 0x7fffffff;
  r.ghi = -1;
#pragma unroll
  for (int x = 0; x < NW; ++x) {
    const double sw = sm.rd[x];
    if (sw > 0.0) {
      if (cw < 0 && run + sw > target) {
        cw = x;
        cb = run;
      }
      lw = x;
      lb = run;
    }
    run += sw;
    r.glo = min(r.glo, sm.ri[x]);
    r.ghi = max(r.ghi, sm.rj[x]);
  }
  r.total = run - base;
  r.crossed = cw >= 0;
  const int ww = cw >= 0 ? cw : lw;
  if (wv == ww) {
    const double c0 = (cw >= 0 ? cb : lb) + inc - ts;  // the running sum before this lane's groups
    const uint64_t bc = __ballot(cw >= 0 && ts > 0.0 && c0 + ts > target);
    const uint64_t bw = __ballot(ts > 0.0);
    const int src = bc ? __ffsll((long long)bc) - 1 : 63 - __clzll((long long)bw);
    if (lane == src) {
      int y = -1, ylast = -1;
      double cl = 0.0, ch = 0.0, ll = 0.0, lh = 0.0;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        double rr = hh ? c0 + (double)s8[0] : c0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float wk = w[hh][k];
          const double rn = rr + (double)wk;
          if (wk > 0.0f) {
            if (y < 0 && cw >= 0 && rn > target) {
              y = e[hh] + k;
              cl = rr;
              ch = rn;
            }
            ylast = e[hh] + k;
            ll = rr;
            lh = rn;
          }
          rr = rn;
        }
      }
      if (y < 0) {  // rounding inside the group, or no crossing at all
        y = ylast;
        cl = ll;
        ch = lh;
      }
      sm.misc[3] = (uint32_t)y;
      sm.rx[0] = cl;
      sm.rx[1] = ch;
    }
  }
  __syncthreads();
  r.y = ww >= 0 ? (int)sm.misc[3] : -1;
  r.clo = sm.rx[0];
  r.chi = sm.rx[1];
  return r;
}

// The residual draw of sequence b at its first rejection n from the span
// sums draw_sum_kernel made (whole work-group).  Wave 0 locates the span
// holding u S from the sums (lane l holding spans [l m, l m + m); `pre`,
// loaded with the records, is lane l's span when there is one span per
// lane), then the work-group draws inside it.  Without residual mass it is
// the rows' own draw, which falls back to q.
template <int DT, bool VEC>
__device__ __forceinline__ Draw draw_spread(const KParams& P, int b, int n, const RowRec& rq, const RowRec& rp,
                                            double u, const DrawSum& pre, SmemSeq<kSeqWaves>& sm, int lane,
                                            int wv) {
  const int D = P.D;
  const RowW wq = row_w(rq), wp = row_w(rp);
  const bool all = __builtin_amdgcn_readfirstlane((int)(wq.T == -kInf && wp.T == -kInf)) != 0;
  const char* qrow = static_cast<const char*>(row_ptr<DT>(P, b, true, n));
  const char* prow = static_cast<const char*>(row_ptr<DT>(P, b, false, n));
  if (wv == 0) {
    const int m = (D + kWave - 1) / kWave;
    double ls = 0.0;
    int lf = 0x7fffffff, ll = -1;
    if (m == 1) {
      ls = pre.s;
      lf = pre.first;
      ll = pre.last;
    } else {
      for (int k = 0; k < m; ++k) {
        const int sp = lane * m + k;
        if (sp < D) {
          const DrawSum d = P.dsums[(size_t)b * D + sp];
          ls += d.s;
          lf = min(lf, d.first);
          ll = max(ll, d.last);
        }
      }
    }
    const double inc = wave_incl_scan(ls, lane);
    const double S = lane63(inc);
    const int nzlo = wave_min_i(lf), nzhi = wave_max_i(ll);
    const double target = u * S;
    // the first lane whose running sum crosses u S (else, u S beyond the
    // rounded total: the last lane with weight), then its span
    const uint64_t bc = __ballot(ls > 0.0 && inc > target);
    const uint64_t bw = __ballot(ls > 0.0);
    const bool beyond = bc == 0;
    const int src = !beyond ? __ffsll((long long)bc) - 1 : bw ? 63 - __clzll((long long)bw) : 0;
    if (lane == src) {
      double run = inc - ls;
      int c = -1, cl = -1;
      double cb = 0.0, lb = 0.0;
      for (int k = 0; k < m; ++k) {
        const int sp = lane * m + k;
        if (sp >= D) break;
        const double sk = m == 1 ? pre.s : P.dsums[(size_t)b * D + sp].s;
        if (sk > 0.0) {
          if (c < 0 && run + sk > target) {
            c = sp;
            cb = run;
          }
          cl = sp;
          lb = run;
        }
        run += sk;
      }
      if (c < 0) {  // beyond, or rounding between the lane's sum and its spans'
        c = cl;
        cb = lb;
      }
      sm.dl_lo = c * kDrawSpan;
      sm.dl_hi = min(P.V, (c + 1) * kDrawSpan);
      sm.dl_base = cb;
      sm.dl_beyond = beyond ? 1 : 0;
    }
    if (lane == 0) {
      sm.dl_S = S;
      sm.dl_nzlo = nzlo;
      sm.dl_nzhi = nzhi;
    }
  }
  __syncthreads();
  const double S = sm.dl_S;
  if (!(S > 0.0)) return draw_from_rows<DT, VEC, kSeqWaves>(P, rq, true, rp, qrow, prow, u, sm, lane, wv, nullptr);
  const int lo = sm.dl_lo, hi = sm.dl_hi, nzlo = sm.dl_nzlo, nzhi = sm.dl_nzhi;
  const bool beyond = sm.dl_beyond != 0;
  const double base = sm.dl_base;
  const RangeDraw r = draw_range<DT, VEC, kSeqWaves>(P, wq, true, wp, all, qrow, prow, lo, hi, base,
                                                     beyond ? kInf : u * S, sm, lane, wv);
  Draw d;
  d.flags = SV_ST_REREAD | SV_ST_LOCATED;
  d.y = r.y;
  if (r.y >= 0) {
    const double plo = (r.crossed ? r.clo : S) / S, phi = (r.crossed ? r.chi : S) / S;
    if (nzlo < d.y && u - plo < kWindow) d.flags |= SV_ST_MARGIN;
    if (nzhi > d.y && phi - u < kWindow) d.flags |= SV_ST_MARGIN;
  } else {
    d.y = 0;
  }
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


// NW waves per work-group: kSeqWaves for small batches (a sequence's draw
// from the rows then has the most waves), 4 for large ones (more sequences
// resident per CU).
// The accept walk and the draw of sequence b, by a work-group of NW waves.
// kCoh: the row records, kept lists and chunk sums were written by other
// work-groups of the running kernel (a fused call's last row of the
// sequence) and are read with coherent loads.
template <int DT, bool VEC, int NW, bool kCoh>
__device__ __forceinline__ void seq_body(const KParams& P, int b, const SeqParams& sp, SmemSeq<NW>& sm) {
  constexpr int NT = NW * kWave;
  const int tid = threadIdx.x, lane = (int)__lane_id();
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  const int Kb = sp.Kb, KM = P.K_max, R = P.R;
  const uint64_t g = P.row_offset + (uint64_t)b;
  const bool greedy = sp.mode == SV_GREEDY;
  // greedy calls may come without draft logits: the rule then needs only
  // the target's argmax (the draft rows' records are not made)
  const bool have_draft = P.draft != nullptr;
  for (int r = tid; r < R; r += NT) {
    const bool used = r <= KM ? r <= Kb : (r - KM - 1 < Kb && have_draft);
    if (used) sm.rows[r] = load_rec<kCoh>(P.rows + (size_t)b * R + r);
  }
  // Loaded with the records by wave 0, for draws that may follow the walk:
  // the span sums of a spread residual draw (lane l: span l) and the chunk
  // sums of target row K_b for a plain bonus draw (lane l: chunk l).
  DrawSum dsp;
  dsp.s = 0.0;
  dsp.first = 0x7fffffff;
  dsp.last = -1;
  ChunkRec crp;
  crp.z = 0.0;
  crp.o = 0.0f;
  crp.pad = 0;
  if (wv == 0) {
    if (NW == kSeqWaves && P.spread && P.D <= kWave && lane < P.D) dsp = P.dsums[(size_t)b * P.D + lane];
    if (P.S <= kWave && lane < P.S) crp = load_rec<kCoh>(P.chunks + ((size_t)b * R + Kb) * P.S + lane);
  }
  // The walk's uniforms depend only on seed, sequence, position and
  // purpose: the last wave draws those of positions 0..63 while the records
  // load.  Greedy rows use none (u p < q with p, q in {0, 1} holds iff q = 1).
  if (!greedy && wv == NW - 1) {
    const int t = lane;
    if (t < Kb) sm.ua[t] = uniform24(P.seed, g, (uint32_t)t, kPurposeAccept);
    if (t <= Kb) sm.ud[t] = uniform24(P.seed, g, (uint32_t)t, t < Kb ? kPurposeResample : kPurposeBonus);
  }
  __syncthreads();

  // Wave 0: the rows' flags, the accept walk, and the draw when it needs no
  // more than the kept list.  The work-group joins only for a draw from the
  // rows.
  if (wv == 0) {
    uint32_t st = 0;
    for (int t = lane; t <= Kb; t += kWave) st |= sm.rows[t].flags;
    if (have_draft)
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
            if (have_draft) p = (float)sm.rows[KM + 1 + t].pid;
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
        const bool have_u = t0 == 0;  // drawn by the last wave (t < 64)
        if (t < Kb) {
          const double q = sm.rows[t].pid;
          const double p = have_draft ? sm.rows[KM + 1 + t].pid : __builtin_nan("");
          if (p == 0.0) s2 |= SV_ST_PZERO;
          if (greedy) {
            rej = !(q > 0.0);
          } else {
            const double ua = have_u ? sm.ua[t] : uniform24(P.seed, g, (uint32_t)t, kPurposeAccept);
            rej = !(ua * p < q);
            // q / p < 1 + w and |u - q / p| < w, multiplied through by p > 0
            if (p > 0.0 && q < p * (1.0 + kWindow) && fabs(ua * p - q) < kWindow * p) s2 |= SV_ST_MARGIN;
          }
        }
        if (!greedy && t <= Kb)
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
      const RowRec& rp = resample && have_draft ? sm.rows[KM + 1 + n] : sm.rows[n];
      if (greedy) {
        const int y = rq.g;
        if (resample && have_draft && rp.g == rq.g) st |= SV_ST_ZERO_RESIDUAL;
        write_tokens(P, b, n, y, st, lane, kWave);
      } else if (rq.flags & kRfListOk) {
        const KeptEntry* kl = P.kept + ((size_t)b * (KM + 1) + n) * (size_t)min(kListMax, P.V);
        const void* prow = resample && have_draft ? row_ptr<DT>(P, b, false, n) : nullptr;
        const Draw d = draw_from_list<DT, kCoh>(rq, resample && have_draft, rp, kl, prow, u, lane);
        write_tokens(P, b, n, d.y, st | d.flags, lane, kWave);
      } else {
        job = 1;
        if (!resample && (rq.flags & kRfChunks) && P.S <= kWave) {
          // a plain bonus draw: the chunk holding u, from the chunk sums
          // (lane l: chunk l; the weights of draw_from_rows), and the work-
          // group draws inside it
          const float c2f = (float)rq.c2;
          const double wc = crp.z > 0.0 ? crp.z * exp2((double)crp.o - (double)rq.M * (double)c2f) / rq.Zs : 0.0;
          const double inc = wave_incl_scan(wc, lane);
          const uint64_t bc = __ballot(wc > 0.0 && inc > u);
          const uint64_t bw = __ballot(wc > 0.0);
          if (bw) {
            job = 2;
            const int c = bc ? __ffsll((long long)bc) - 1 : 63 - __clzll((long long)bw);
            const double base = bc ? lane_at(inc - wc, c) : 0.0;  // (u beyond the rounded total: the last token with weight)
            if (lane == 0) {
              sm.dl_lo = c * P.L;
              sm.dl_hi = min(P.V, c * P.L + P.L);
              sm.dl_base = base;
              sm.dl_beyond = bc ? 0 : 1;
            }
          }
        }
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
  const uint32_t job = sm.misc[2];
  if (job == 0u) return;
  // draw from the rows (plain rows, or a kept set not held as a list)
  const int n = (int)sm.misc[0];
  uint32_t st = sm.misc[1];
  const double u = sm.rx[0];
  const bool resample = n < Kb;
  const RowRec rq = sm.rows[n];
  const RowRec rp = resample ? sm.rows[KM + 1 + n] : rq;
  __syncthreads();  // sm.misc / sm.rx are reused by the draw
  if (job == 2u) {
    // a plain bonus draw inside the chunk located by wave 0
    const RowW wq = row_w(rq);
    const bool all = __builtin_amdgcn_readfirstlane((int)(wq.T == -kInf)) != 0;
    const double base = sm.dl_base;
    const RangeDraw r =
        draw_range<DT, VEC, NW>(P, wq, false, wq, all, static_cast<const char*>(row_ptr<DT>(P, b, true, n)), nullptr,
                                sm.dl_lo, sm.dl_hi, 0.0, sm.dl_beyond ? kInf : u - base, sm, lane, wv);
    if (r.y >= 0) {
      uint32_t fl = SV_ST_REREAD | SV_ST_LOCATED;
      const double plo = base + (r.crossed ? r.clo : r.total), phi = base + (r.crossed ? r.chi : r.total);
      if (r.glo < r.y && u - plo < kWindow) fl |= SV_ST_MARGIN;
      if (r.ghi > r.y && phi - u < kWindow) fl |= SV_ST_MARGIN;
      write_tokens(P, b, n, r.y, st | fl, tid, NT);
      return;
    }
    __syncthreads();  // (no weight in the chunk after all: the draw below)
  }
  // a residual draw with the span sums made before this kernel, or the
  // work-group's own pass over the rows
  Draw d;
  if constexpr (NW == kSeqWaves) {
    if (P.spread && resample) d = draw_spread<DT, VEC>(P, b, n, rq, rp, u, dsp, sm, lane, wv);
  }
  if (!(NW == kSeqWaves && P.spread && resample))
    d = draw_from_rows<DT, VEC, NW, kCoh>(P, rq, resample, rp, static_cast<const char*>(row_ptr<DT>(P, b, true, n)),
                                    resample ? static_cast<const char*>(row_ptr<DT>(P, b, false, n)) : nullptr, u,
                                    sm, lane, wv, P.chunks + ((size_t)b * R + n) * P.S);
  write_tokens(P, b, n, d.y, st | d.flags, tid, NT);
}

template <int DT, bool VEC, int NW>
__global__ __launch_bounds__(NW * kWave) void seq_kernel(const KParams P) {
  warm_kernel_args();
  __shared__ SmemSeq<NW> sm;
  const int b = P.b_base + (int)blockIdx.x;
  const SeqParams sp = load_params(P, b);
  if (!sp.valid) {
    write_error(P, b, SV_ST_PARAM, (int)threadIdx.x, NW * kWave);
    return;
  }
  seq_body<DT, VEC, NW, false>(P, b, sp, sm);
}

// start / stop: events recorded on the kernel's own dispatch (NULL: none).
template <int DT, bool VEC, bool FUSE>
void launch_rows_as(const KParams& p, int mode, dim3 grid, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  const dim3 block(kThreads);
  switch (mode) {
    case SV_PLAIN:  // (plain calls are not fused)
      if constexpr (!FUSE)
        hipExtLaunchKernelGGL((row_kernel<DT, VEC, SV_PLAIN, false>), grid, block, 0, stream, start, stop, 0, p);
      break;
    case SV_TOPK: hipExtLaunchKernelGGL((row_kernel<DT, VEC, SV_TOPK, FUSE>), grid, block, 0, stream, start, stop, 0, p); break;
    case SV_TOPP: hipExtLaunchKernelGGL((row_kernel<DT, VEC, SV_TOPP, FUSE>), grid, block, 0, stream, start, stop, 0, p); break;
    case SV_GREEDY: hipExtLaunchKernelGGL((row_kernel<DT, VEC, SV_GREEDY, FUSE>), grid, block, 0, stream, start, stop, 0, p); break;
    default:
      if constexpr (!FUSE)
        hipExtLaunchKernelGGL((row_kernel<DT, VEC, kAnyMode, false>), grid, block, 0, stream, start, stop, 0, p);
      break;
  }
}

template <int DT, bool VEC>
void launch_rows(const KParams& p, int mode, dim3 grid, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  if (p.fuse) launch_rows_as<DT, VEC, true>(p, mode, grid, stream, start, stop);
  else launch_rows_as<DT, VEC, false>(p, mode, grid, stream, start, stop);
}

template <int DT, bool VEC>
hipError_t launch_all(const KParams& p, int nseq, hipStream_t stream, hipEvent_t* ev) {
  // one row-kernel instance: the default mode's, or the one holding every
  // path when the call gives a mode per sequence
  // A launch of one to three rows per CU streams the rows beyond a whole
  // number per CU in parts, one per CU (calls with one filter of plain,
  // nucleus or greedy, whose row kernels hold three work-groups per CU;
  // top-k lists cut per part would not fit the merge).
  KParams q = p;
  const size_t rows = (size_t)nseq * (p.draft ? p.R : p.K_max + 1);
  q.full = (int)rows;
  q.parts = 1;
  if (VEC && !p.mode && p.dmode != SV_TOPK) q.parts = row_split(rows, p.S, &q.full);
  q.nsplit = (int)((rows - (size_t)q.full) * q.parts);
  const size_t wgs = (size_t)q.full + (size_t)q.nsplit;
  q.prio = wgs > 2 * (size_t)kRowCUs && wgs <= 3 * (size_t)kRowCUs ? 1 : 0;
  // The sequence step is fused into the row kernel for launches of one
  // round of one to three work-groups per CU (one filter): there it runs
  // while other rows stream, and the second launch is saved.  Larger
  // launches keep the sequence kernel (its smaller work-groups hold more
  // sequences per CU than a row work-group does), and so do plain calls:
  // their first rejection always draws from the rows, which the 8-wave
  // sequence kernel does faster than a row work-group's 4 waves.
  q.fuse = p.fuse && !p.mode && p.dmode != SV_PLAIN && wgs > (size_t)kRowCUs && wgs <= 3 * (size_t)kRowCUs &&
                   nseq <= kMaxFusedSeq
               ? 1
               : 0;
  const dim3 grid((unsigned)wgs);
  launch_rows<DT, VEC>(q, p.mode ? kAnyMode : p.dmode, grid, stream, ev ? ev[0] : nullptr, ev ? ev[1] : nullptr);
  hipEvent_t seq_start = ev ? ev[2] : nullptr;
  if (q.fuse) {
    // the sequence step ran in the row kernel: the second stage is empty
    if (ev) {
      (void)hipEventRecord(ev[2], stream);
      (void)hipEventRecord(ev[3], stream);
    }
    return hipSuccess;
  }
  if (p.spread) {
    // the span sums of the residual draws over the whole chip, then the
    // walk and draws
    hipExtLaunchKernelGGL((draw_sum_kernel<DT, VEC>), dim3((unsigned)((size_t)nseq * p.D)), dim3(kThreads), 0,
                          stream, seq_start, nullptr, 0, p);
    seq_start = nullptr;
  }
  // several sequences per CU: smaller work-groups, more of them resident
  if (nseq >= kSmallSeqWgMin)
    hipExtLaunchKernelGGL((seq_kernel<DT, VEC, 4>), dim3((unsigned)nseq), dim3(4 * kWave), 0, stream, seq_start,
                          ev ? ev[3] : nullptr, 0, p);
  else
    hipExtLaunchKernelGGL((seq_kernel<DT, VEC, kSeqWaves>), dim3((unsigned)nseq), dim3(kSeqThreads), 0, stream,
                          seq_start, ev ? ev[3] : nullptr, 0, p);
  return hipSuccess;
}

}  // namespace


namespace {

// Read-only streaming probe with the streaming pass's access pattern and
// non-temporal loads: each wave reads one 8 KB block as 8 x 16-byte
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

// Read-rate sweep: work-group g reads blocks [g n / G, (g + 1) n / G) of
// NL x 64 vectors each, its waves taking the blocks in turn, with the next
// block's loads in flight while the current one is folded.
template <int NL>
__global__ __launch_bounds__(kThreads) void stream_sweep_kernel(const uint4* data, size_t nblocks, uint32_t* out) {
  const int lane = (int)__lane_id();
  const int wv = (int)(threadIdx.x / kWave);
  const size_t G = gridDim.x;
  const size_t b0 = nblocks * blockIdx.x / G, b1 = nblocks * (blockIdx.x + 1) / G;
  uint4 a[NL], c[NL];
  auto issue = [&](uint4 (&v)[NL], size_t b) {
    const uint4* base = data + (b < b1 ? b : b1 - 1) * (size_t)(NL * kWave);  // (a block past the range: its last, again)
#pragma unroll
    for (int i = 0; i < NL; ++i) v[i] = load_stream(&base[i * kWave + lane]);
  };
  uint32_t x = 0;
  auto fold = [&](const uint4 (&v)[NL]) {
#pragma unroll
    for (int i = 0; i < NL; ++i) x ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  };
  size_t b = b0 + wv;
  if (b < b1) {
    issue(a, b);
    while (true) {
      issue(c, b + kRowWaves);
      fold(a);
      b += kRowWaves;
      if (b >= b1) break;
      issue(a, b + kRowWaves);
      fold(c);
      b += kRowWaves;
      if (b >= b1) break;
    }
  }
  if (x == 0x9e3779b9u) out[0] = x;
}

hipError_t launch_stream_sweep(const void* data, size_t bytes, int loads_per_lane, int waves_per_cu, uint32_t* out,
                               hipStream_t stream) {
  const size_t nblocks = bytes / ((size_t)loads_per_lane * kWave * sizeof(uint4));
  if (nblocks == 0) return hipSuccess;
  const dim3 grid((unsigned)(256 * waves_per_cu / kRowWaves)), block(kThreads);
  const uint4* d = static_cast<const uint4*>(data);
  switch (loads_per_lane) {
    case 4: hipLaunchKernelGGL(stream_sweep_kernel<4>, grid, block, 0, stream, d, nblocks, out); break;
    case 8: hipLaunchKernelGGL(stream_sweep_kernel<8>, grid, block, 0, stream, d, nblocks, out); break;
    default: hipLaunchKernelGGL(stream_sweep_kernel<16>, grid, block, 0, stream, d, nblocks, out); break;
  }
  return hipGetLastError();
}

hipError_t launch_stream_probe(const void* data, size_t bytes, uint32_t* out, hipStream_t stream) {
  const size_t nblocks = bytes / (kLoads * kWave * sizeof(uint4));
  if (nblocks == 0) return hipSuccess;
  const size_t wg = (nblocks + kThreads / kWave - 1) / (kThreads / kWave);
  hipLaunchKernelGGL(stream_probe_kernel, dim3((unsigned)wg), dim3(kThreads), 0, stream,
                     static_cast<const uint4*>(data), nblocks, out);
  return hipGetLastError();
}

namespace {
__global__ __launch_bounds__(256) void philox_words_kernel(uint64_t seed, const uint64_t* g, const uint32_t* t,
                                                           const uint32_t* purpose, int64_t n, uint32_t* out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) out[i] = philox_word0(seed, g[i], t[i], purpose[i]);
}
}  // namespace

hipError_t launch_philox_words(uint64_t seed, const uint64_t* g, const uint32_t* t, const uint32_t* purpose,
                               int64_t n, uint32_t* out, hipStream_t stream) {
  for (int64_t i0 = 0; i0 < n; i0 += (int64_t)1 << 30) {  // grids of at most 2^30 work-items
    const int64_t m = n - i0 < ((int64_t)1 << 30) ? n - i0 : ((int64_t)1 << 30);
    hipLaunchKernelGGL(philox_words_kernel, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, stream, seed, g + i0,
                       t + i0, purpose + i0, m, out + i0);
  }
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
