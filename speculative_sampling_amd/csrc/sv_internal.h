// Internal layout shared by the host code and the gfx950 kernels of
// libspec_verify.  Not part of the public ABI (include/spec_verify.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "spec_verify.h"

namespace sv {

// Work-group of the row kernel: 4 wave64s stream one logit row.
constexpr int kRowWaves = 4;
constexpr int kThreads = 64 * kRowWaves;
// Each wave streams its share of a row in chunks: every lane keeps kLoads
// 16-byte vectors of a chunk in registers (32 VGPRs), 64 bf16 or 32 fp32
// logits, so a chunk (8 KB) holds 4096 bf16 / 2048 fp32 logits.
constexpr int kLoads = 8;
// Candidate vectors (the 16-byte logit vectors that may hold a token of a
// top-k / nucleus kept set) one wave can keep in LDS for its share of a row.
constexpr int kCandVecs = 256;
// Largest kept set of a target row that is written out as a list, so that
// the final draw needs no second read of the logit rows.
constexpr int kListMax = 512;
// Waves of the per-sequence kernel (accept walk and final draw) for calls
// of fewer than kSmallSeqWgMin sequences; 4 waves for larger calls.
constexpr int kSeqWaves = 8;
constexpr int kSmallSeqWgMin = 1024;
constexpr int kMaxK = 64;
constexpr int kMaxVocab = 1 << 22;

inline int chunk_capacity(int dtype) { return 64 * kLoads * (dtype == SV_BF16 ? 8 : 4); }

// Per-(row, chunk) softmax sums of a plain target row: its bonus draw
// locates the chunk that holds its target from them.
struct ChunkRec {
  double z;     // sum over the chunk of 2^(x c2 - o)  (0: no finite logit)
  float o;      // exponent offset of the chunk's terms
  int32_t pad;
};
constexpr uint32_t kCfNonFinite = 1u;

// One logit row (one model at one position of one sequence) after the row
// kernel: everything the accept walk and the final draw need.
struct RowRec {
  float M;          // row maximum (raw logit)
  float T;          // kept set is {x >= T}; -inf when every token is kept
  double c2;        // log2(e) / temperature
  double Zs;        // kept mass: sum_{x >= T} 2^((x - M) * c2)
  double pid;       // probability of this row's draft token (NaN if none)
  int32_t g;        // greedy argmax
  int32_t n_keep;   // |{x >= T}|, -1 if not counted
  uint32_t flags;   // SV_ST_* error/info bits of the row, plus kRf* below
  int32_t pad;
};
// The row's kept set is stored, in vocabulary order, in its KeptEntry list.
constexpr uint32_t kRfListOk = 1u << 16;
// The row's chunk records (ChunkRec) were written.
constexpr uint32_t kRfChunks = 1u << 17;

// One token of a target row's kept set: vocabulary index and the target's
// logit.
struct KeptEntry {
  int32_t idx;
  float xq;
};

// Residual draws spread over the chip: a sequence whose first rejection n
// (< K_b) needs the rows themselves (plain rows, a kept set not listed)
// draws from (q_n - p_n)+ in vocabulary order.  Before the sequence
// kernel, one work-group per kDrawSpan tokens of each sequence repeats the
// accept walk and, for such a sequence, sums its span's weights into a
// DrawSum; the sequence kernel then locates the span holding the target
// and draws in it.  (Spans of 4096 tokens measured faster than 8192 and
// 2048 at the headline shape in plain mode.)
constexpr int kDrawSpan = 4096;
struct DrawSum {
  double s;       // sum of the span's weights, fp32 groups of 8 added in fp64
  int32_t first;  // first token of the span's first group of 8 with weight (INT32_MAX: none)
  int32_t last;   // last token of its last group of 8 with weight (-1: none)
};

// Balanced launches.  The nucleus, plain and greedy row kernels hold at
// least three work-groups per CU.  A launch of between one and three rows
// per CU (kRowCUs CUs), not a whole number of them, would leave some CUs a
// row more than the others; instead the first k kRowCUs rows (k = 1, 2)
// are streamed whole and each remaining row is split into `parts`
// contiguous ranges of chunks, one work-group each, so that every CU
// streams about the same bytes.  A part
// leaves its waves' records and candidate lists in a PartHdr and the part
// lists; the last part of a row to arrive (a counter per row) merges them
// and finishes the row.
constexpr int kRowCUs = 256;
constexpr int kMaxParts = 4;
// The split of a launch of `rows` rows of S chunks: rows [0, *full) whole,
// the rest in the returned number of parts each (1: no split).
inline int row_split(size_t rows, int S, int* full) {
  *full = (int)rows;
  if (rows <= (size_t)kRowCUs || rows >= 3 * (size_t)kRowCUs || rows % kRowCUs == 0) return 1;
  const size_t whole = rows / kRowCUs * kRowCUs;
  const int extra = (int)(rows - whole);
  int p = kRowCUs / extra;
  p = p < kMaxParts ? p : kMaxParts;
  p = p < S / kRowWaves ? p : S / kRowWaves;  // at least one chunk per wave of every part
  if (p < 2) return 1;
  *full = (int)whole;
  return p;
}
// What one part's waves found (written with coherent stores).
struct PartWave {
  double z;        // the wave's softmax sum (see the row kernel's WaveRec)
  float m, o;      // largest logit; exponent offset of z
  int32_t arg;     // greedy: lowest index holding m
  uint32_t flags;  // kCfNonFinite
  int32_t ncand;   // candidate vectors listed, -1 after an overflow
  float ucut;      // the largest listing cut used
  float pub;       // the part's running maximum (nucleus) at its end
  int32_t pad;
};
struct PartHdr {
  PartWave w[kRowWaves];
};
// Split rows per launch: at most kRowCUs parts (extra rows x parts).
constexpr int kMaxSplitRows = kRowCUs / 2;
// Fused calls: calls whose residual draws are not spread over the chip run
// the per-sequence accept walk and draw in the row kernel, by the last row
// of each sequence to finish (a counter per sequence), instead of in a
// second kernel.  A fused launch holds at most three row work-groups per CU,
// each of at least one row of its own sequence: at most kMaxFusedSeq sequences.
constexpr int kMaxFusedSeq = 3 * kRowCUs;

struct KParams {
  int32_t B, K_max, V, R, S, L;
  int32_t b_base, b_end;  // sequences [b_base, b_end) of this launch
  const void* target;
  const void* draft;
  const int32_t* tokens;
  const int32_t* kpr;
  const uint8_t* mode;
  const float* temp;
  const int32_t* topk;
  const float* topp;
  int32_t dmode;
  float dtemp;
  int32_t dtopk;
  float dtopp;
  uint64_t seed;
  uint64_t row_offset;
  int32_t* accepted;
  int32_t* out_tokens;
  uint32_t* status;
  float* diag;
  ChunkRec* chunks;  // [B][R][S]  (plain target rows)
  RowRec* rows;      // [B][R]
  KeptEntry* kept;   // [B][K_max + 1][min(kListMax, V)]  (target rows)
  DrawSum* dsums;    // [B][D]  (spread draws)
  int32_t D;         // spans of kDrawSpan tokens per row
  int32_t spread;    // residual draws from the rows go to the draw kernels
  int32_t full;      // rows [0, full) of the launch streamed whole (row_split)
  int32_t parts;     // work-groups per remaining row
  int32_t nsplit;    // the part work-groups, (rows - full) x parts, launched first
  int32_t prio;      // waves lower their issue priority as they progress (launches of one round)
  int32_t fuse;      // the sequence step runs in the row kernel (the last row of each sequence); set per launch
  int32_t* scount;   // [kMaxFusedSeq] arrivals per sequence of a fused launch (0 between calls)
  int32_t* pcount;   // [kMaxSplitRows] arrivals per split row (0 between calls)
  PartHdr* phdr;     // [kRowCUs] part records
  uint4* pvec;       // [kRowCUs][kRowWaves][kCandVecs] listed vectors
  uint2* pik;        // [kRowCUs][kRowWaves][kCandVecs] (first index, key bits)
};

// Enqueues the kernels of one call for sequences
// [p.b_base, p.b_base + nseq): the row kernel (the default mode's instance,
// or the one holding every mode's path when the call gives a mode per
// sequence), then the per-sequence accept walk and draw.  When ev is not
// NULL, ev[0] / ev[1] mark the start and end of the row kernel, ev[2] /
// ev[3] those of the sequence kernel, each recorded on the kernel's own
// dispatch.
hipError_t launch_verify(const KParams& p, int dtype, bool vec, int nseq, hipStream_t stream,
                         hipEvent_t* ev = nullptr);
// Reads the first bytes / 8192 whole 8 KB blocks of data once (see spec_verify_stream_probe).
hipError_t launch_stream_probe(const void* data, size_t bytes, uint32_t* out, hipStream_t stream);
// Philox word 0 for n counters (see spec_verify_philox_words).
hipError_t launch_philox_words(uint64_t seed, const uint64_t* g, const uint32_t* t, const uint32_t* purpose,
                               int64_t n, uint32_t* out, hipStream_t stream);
// One point of the read-rate sweep (see spec_verify_stream_probe_sweep).
hipError_t launch_stream_sweep(const void* data, size_t bytes, int loads_per_lane, int waves_per_cu, uint32_t* out,
                               hipStream_t stream);

}  // namespace sv
