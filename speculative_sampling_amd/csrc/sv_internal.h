// Internal layout shared by the host code and the gfx950 kernels of
// libspec_verify.  Not part of the public ABI (include/spec_verify.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "spec_verify.h"

namespace sv {

// Work-group shape of every kernel: 4 wave64s.
constexpr int kThreads = 256;
// The streaming kernel gives each wave (64 lanes) one chunk of a row; each
// lane keeps kLoads 16-byte vectors of it in registers (64 VGPRs): 128 bf16
// or 64 fp32 logits, so a chunk holds at most 8192 bf16 / 4096 fp32 logits.
constexpr int kLoads = 16;
// Candidate list capacity per chunk, in 16-byte logit vectors: the vectors
// that may hold a token near the maximum, kept for the top-k / nucleus
// threshold search (fewer per chunk when a row has many chunks).
constexpr int kCandVecs = 256;
// Largest kept set the final draw takes from the merged kept list without
// re-reading the logit rows.
constexpr int kListMax = 512;
// Waves of the per-sequence kernel (one logit row each); sequences of more
// rows keep their kept lists in global memory.
constexpr int kSeqWaves = 12;
constexpr int kMaxK = 64;
constexpr int kMaxVocab = 1 << 22;

inline int chunk_capacity(int dtype) { return 64 * kLoads * (dtype == SV_BF16 ? 8 : 4); }

// Per-(row, chunk) partial results written by the streaming kernel.
struct ChunkRec {
  float m;         // chunk maximum of the raw logits (-inf if none is finite)
  float cut;       // every token of the chunk with logit >= cut (and > -inf) lies
                   // in a vector of the chunk's candidate list; +inf when the
                   // list is incomplete
  double z;        // sum over the chunk of 2^((x - m) * c2)   (plain, nucleus)
  int32_t cnt;     // candidate vectors stored
  int32_t arg;     // lowest index whose logit equals m      (greedy)
  uint32_t flags;  // kCfNonFinite
  float o;         // listed vectors' keys are terms 2^(x c2 - o) (nucleus)
};
constexpr uint32_t kCfNonFinite = 1u;

// Per logit row (one model at one position of one sequence) after merging;
// held in LDS by the sequence kernel.
struct RowRec {
  float M;          // row maximum (raw logit)
  float T;          // kept set is {x >= T}; -inf for plain
  double c2;        // log2(e) / temperature
  double Zs;        // kept mass: sum_{x >= T} 2^((x - M) * c2)
  double pid;       // probability of this row's draft token (NaN if none)
  int32_t g;        // greedy argmax
  int32_t n_keep;   // |{x >= T}|, -1 if not counted
  uint32_t flags;   // SV_ST_* error/info bits of the row, plus kRf* below
  int32_t pad;
};
// The row's kept set is stored, in vocabulary order with its probabilities,
// in the row's KeptEntry list.
constexpr uint32_t kRfListOk = 1u << 16;

// One token of a target row's kept set: vocabulary index and probability.
struct KeptEntry {
  int32_t idx;
  int32_t pad;
  double q;
};

struct KParams {
  int32_t B, K_max, V, R, S, L;
  int32_t cap;  // candidate vectors per chunk
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
  ChunkRec* chunks;
  int2* cent;      // [row][chunk][cap] candidate vectors: first logit index and key
  KeptEntry* kept;  // [rows][kListMax]
};

// Enqueues the kernels of one call for sequences
// [p.b_base, p.b_base + nseq): the streaming chunk pass (the default mode's
// instance, or the one holding every mode's path when the call gives a mode
// per sequence), then the per-sequence merge, accept walk and draw.
// When ev is not NULL, ev[0] / ev[1] mark the start and end of the streaming
// kernel, ev[2] / ev[3] those of the sequence kernel, each recorded on the
// kernel's own dispatch.
hipError_t launch_verify(const KParams& p, int dtype, bool vec, int nseq, hipStream_t stream,
                         hipEvent_t* ev = nullptr);
// Reads the first bytes / 16384 whole 16 KB blocks of data once (see spec_verify_stream_probe).
hipError_t launch_stream_probe(const void* data, size_t bytes, uint32_t* out, hipStream_t stream);

}  // namespace sv
