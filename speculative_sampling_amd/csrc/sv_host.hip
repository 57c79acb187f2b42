// Host side of libspec_verify: the C ABI declared in include/spec_verify.h.
//
// create  allocates the device workspace once (chunk records, row records,
//         kept lists);
// run     validates on the host, then enqueues the kernels of the step for
//         batches of at most kMaxSeqPerLaunch sequences and kMaxRowsPerLaunch
//         rows on the caller's stream;
// destroy synchronises the device if the handle has run, then frees.
// run_static runs the same kernels with the workspace in a static device
//         array (no allocation at all), for callers that cannot allocate.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "spec_verify.h"
#include "sv_internal.h"

struct sv_handle_s {
  sv_config cfg;
  void* ws;
  size_t ws_bytes;
  bool has_run;  // some run was enqueued (or captured): destroy waits for the device
  // stage timing (spec_verify_profile_begin / _end)
  std::vector<hipEvent_t> prof;
  int prof_max, prof_next;
};

namespace {

thread_local std::string g_last_error;
// A dispatch counts its work-items in 32 bits.  Per launch: at most 2^23
// rows (row-kernel work-groups of kThreads: 2^31 work-items) and 2^22
// sequences (work-groups of kSeqWaves waves: 2^31 work-items).
constexpr size_t kMaxRowsPerLaunch = (size_t)1 << 23;
constexpr size_t kMaxSeqPerLaunch = (size_t)1 << 22;
static_assert(kMaxRowsPerLaunch * sv::kThreads < ((size_t)1 << 32), "row grid");
static_assert(kMaxSeqPerLaunch * sv::kSeqWaves * 64 < ((size_t)1 << 32), "sequence grid");

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

struct Geometry {
  int S, L, R_max, D;
  size_t off_pcount, off_scount, off_chunks, off_rows, off_kept, off_dsums, off_phdr, off_pvec, off_pik, total;
};

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int check_config(const sv_config* cfg) {
  if (!cfg) return fail(SV_EINVAL, "config is NULL");
  if (cfg->dtype != SV_F32 && cfg->dtype != SV_BF16) return fail(SV_EDTYPE, "unknown dtype");
  if (cfg->vocab < 1 || cfg->vocab > sv::kMaxVocab) return fail(SV_EINVAL, "vocab must be in [1, 2^22]");
  if (cfg->max_batch < 1) return fail(SV_EINVAL, "max_batch must be >= 1");
  if (cfg->max_k < 0 || cfg->max_k > sv::kMaxK) return fail(SV_EINVAL, "max_k must be in [0, 64]");
  if (cfg->device < 0) return fail(SV_EINVAL, "device must be >= 0");
  return SV_OK;
}

Geometry geometry(const sv_config* cfg) {
  Geometry g;
  const int V = cfg->vocab;
  const int chunk_cap = sv::chunk_capacity(cfg->dtype);
  // whole chunks of chunk_cap logits, the row's remainder in the last one
  g.S = (V + chunk_cap - 1) / chunk_cap;
  g.L = chunk_cap;
  g.R_max = 2 * cfg->max_k + 1;
  const size_t rows = (size_t)cfg->max_batch * g.R_max;
  const size_t target_rows = (size_t)cfg->max_batch * (cfg->max_k + 1);
  size_t off = 0;
  // the arrival counters of split rows come first, at the same place in
  // every layout: each call leaves them at zero
  g.off_pcount = off;
  off = align_up(off + sv::kMaxSplitRows * sizeof(int32_t), 256);
  g.off_scount = off;  // (also at a fixed place: the sequence counters of fused calls)
  off = align_up(off + sv::kMaxFusedSeq * sizeof(int32_t), 256);
  g.off_chunks = off;
  off = align_up(off + rows * g.S * sizeof(sv::ChunkRec), 256);
  g.off_rows = off;
  off = align_up(off + rows * sizeof(sv::RowRec), 256);
  g.off_kept = off;
  off = align_up(off + target_rows * std::min(sv::kListMax, V) * sizeof(sv::KeptEntry), 256);
  g.D = (V + sv::kDrawSpan - 1) / sv::kDrawSpan;
  g.off_dsums = off;
  off = align_up(off + (size_t)cfg->max_batch * g.D * sizeof(sv::DrawSum), 256);
  // part records of split rows (only launches of 1 to 3 rows per CU split)
  const size_t n_parts = rows > (size_t)sv::kRowCUs && g.S >= 2 * sv::kRowWaves ? sv::kRowCUs : 0;
  g.off_phdr = off;
  off = align_up(off + n_parts * sizeof(sv::PartHdr), 256);
  g.off_pvec = off;
  off = align_up(off + n_parts * sv::kRowWaves * sv::kCandVecs * sizeof(uint4), 256);
  g.off_pik = off;
  off = align_up(off + n_parts * sv::kRowWaves * sv::kCandVecs * sizeof(uint2), 256);
  g.total = off;
  return g;
}

bool finite_pos(float x) { return std::isfinite(x) && x > 0.0f; }

// 16-byte vector loads need every row start on a 16-byte boundary.
bool vector_loads(const sv_config& cfg, const sv_args* a) {
  const int es = cfg.dtype == SV_BF16 ? 2 : 4;
  return ((size_t)cfg.vocab * es) % 16 == 0 && (reinterpret_cast<uintptr_t>(a->target_logits) % 16) == 0 &&
         (a->K_max == 0 || (reinterpret_cast<uintptr_t>(a->draft_logits) % 16) == 0);  // NULL is aligned
}

}  // namespace

extern "C" {

const char* spec_verify_last_error(void) { return g_last_error.c_str(); }

uint64_t spec_verify_workspace_bytes(const sv_config* cfg) {
  if (check_config(cfg) != SV_OK) return 0;
  return geometry(cfg).total;
}

int spec_verify_validate(const sv_config* cfg, const sv_args* a) {
  int rc = check_config(cfg);
  if (rc != SV_OK) return rc;
  if (!a) return fail(SV_EINVAL, "args is NULL");
  if (a->B < 0) return fail(SV_EINVAL, "B must be >= 0");
  if (a->K_max < 0) return fail(SV_EINVAL, "K_max must be >= 0");
  if (a->B > cfg->max_batch) return fail(SV_ECAPACITY, "B exceeds max_batch");
  if (a->K_max > cfg->max_k) return fail(SV_ECAPACITY, "K_max exceeds max_k");
  if (a->B == 0) return SV_OK;
  if (!a->target_logits) return fail(SV_EINVAL, "target_logits is NULL");
  if (a->K_max > 0 && !a->draft_tokens) return fail(SV_EINVAL, "draft_tokens is required when K_max > 0");
  // greedy verification needs only the target's argmax: the draft's logits
  // may be left out when every row is greedy
  if (a->K_max > 0 && !a->draft_logits && (a->mode || a->default_mode != SV_GREEDY))
    return fail(SV_EINVAL, "draft_logits is required when K_max > 0 (unless every row is greedy)");
  if (!a->accepted || !a->out_tokens) return fail(SV_EINVAL, "accepted and out_tokens are required");
  // Rows that are not whole 16-byte vectors (V * element size not a
  // multiple of 16, or a logit buffer not 16-byte aligned) are streamed
  // element by element, which is supported for rows of one chunk only.
  if (!vector_loads(*cfg, a) && cfg->vocab > sv::chunk_capacity(cfg->dtype))
    return fail(SV_EINVAL,
                "rows that are not whole 16-byte vectors (V * element size a multiple of 16, logit buffers "
                "16-byte aligned) are supported only up to 4096 bf16 / 2048 fp32 logits");
  // Defaults are checked only where some row can use them.
  if (!a->mode && (a->default_mode < SV_PLAIN || a->default_mode > SV_GREEDY))
    return fail(SV_EINVAL, "default_mode is not an sv_mode");
  const bool any_mode = a->mode != nullptr;
  const int dm = a->default_mode;
  if (!a->temperature && (any_mode || dm != SV_GREEDY) && !finite_pos(a->default_temperature))
    return fail(SV_EINVAL, "default_temperature must be finite and > 0");
  if (!a->top_k && (any_mode || dm == SV_TOPK) &&
      (a->default_top_k < 1 || a->default_top_k > cfg->vocab))
    return fail(SV_EINVAL, "default_top_k must be in [1, V]");
  if (!a->top_p && (any_mode || dm == SV_TOPP) &&
      !(a->default_top_p > 0.0f && a->default_top_p <= 1.0f))
    return fail(SV_EINVAL, "default_top_p must be in (0, 1]");
  return SV_OK;
}

int spec_verify_create(sv_handle_t* out, const sv_config* cfg) {
  if (!out) return fail(SV_EINVAL, "out is NULL");
  *out = nullptr;
  int rc = check_config(cfg);
  if (rc != SV_OK) return rc;
  int prev = 0;
  if (hipGetDevice(&prev) != hipSuccess) return fail(SV_EHIP, "hipGetDevice failed");
  if (hipSetDevice(cfg->device) != hipSuccess) return fail(SV_EHIP, "hipSetDevice failed");
  Geometry g = geometry(cfg);
  sv_handle_s* h = new (std::nothrow) sv_handle_s();
  if (!h) {
    (void)hipSetDevice(prev);
    return fail(SV_ENOMEM, "host allocation failed");
  }
  h->cfg = *cfg;
  h->ws_bytes = g.total;
  hipError_t e = hipMalloc(&h->ws, g.total);
  if (e != hipSuccess) {
    delete h;
    (void)hipSetDevice(prev);
    return fail(SV_ENOMEM, std::string("hipMalloc of workspace failed: ") + hipGetErrorString(e));
  }
  // the arrival counters of split rows start at zero (each call leaves them so)
  e = hipMemset(static_cast<char*>(h->ws) + g.off_pcount, 0, g.off_chunks - g.off_pcount);  // (and the sequence counters)
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    (void)hipFree(h->ws);
    delete h;
    (void)hipSetDevice(prev);
    return fail(SV_EHIP, std::string("workspace initialisation failed: ") + hipGetErrorString(e));
  }
  h->has_run = false;
  h->prof_max = h->prof_next = 0;
  (void)hipSetDevice(prev);
  *out = h;
  return SV_OK;
}

namespace {

// The kernel parameters of one call: the caller's arguments and the
// workspace laid out by geometry g at ws.
sv::KParams make_params(const sv_config& cfg, const Geometry& g, void* ws, const sv_args* a) {
  sv::KParams p;
  p.B = a->B;
  p.K_max = a->K_max;
  p.V = cfg.vocab;
  p.R = 2 * a->K_max + 1;
  p.S = g.S;
  p.L = g.L;
  p.b_base = 0;
  p.b_end = 0;
  p.target = a->target_logits;
  p.draft = a->K_max > 0 ? a->draft_logits : nullptr;
  p.tokens = a->draft_tokens;
  p.kpr = a->k_per_row;
  p.mode = a->mode;
  p.temp = a->temperature;
  p.topk = a->top_k;
  p.topp = a->top_p;
  p.dmode = a->default_mode;
  p.dtemp = a->default_temperature;
  p.dtopk = a->default_top_k;
  p.dtopp = a->default_top_p;
  p.seed = a->seed;
  p.row_offset = a->row_offset;
  p.accepted = a->accepted;
  p.out_tokens = a->out_tokens;
  p.status = a->row_status;
  p.diag = a->diag;
  char* base = static_cast<char*>(ws);
  p.chunks = reinterpret_cast<sv::ChunkRec*>(base + g.off_chunks);
  p.rows = reinterpret_cast<sv::RowRec*>(base + g.off_rows);
  p.kept = reinterpret_cast<sv::KeptEntry*>(base + g.off_kept);
  p.dsums = reinterpret_cast<sv::DrawSum*>(base + g.off_dsums);
  p.D = g.D;
  p.full = 0;  // set per launch
  p.parts = 1;
  p.nsplit = 0;
  p.prio = 0;
  p.scount = reinterpret_cast<int32_t*>(base + g.off_scount);
  p.pcount = reinterpret_cast<int32_t*>(base + g.off_pcount);
  p.phdr = reinterpret_cast<sv::PartHdr*>(base + g.off_phdr);
  p.pvec = reinterpret_cast<uint4*>(base + g.off_pvec);
  p.pik = reinterpret_cast<uint2*>(base + g.off_pik);
  // Residual draws from the rows are spread over the chip when the call
  // may hold plain rows (their first rejection always needs the rows);
  // other calls draw the rare ones in the sequence kernel.
  // (only where the sequence kernel alone would leave most CUs idle: fewer
  // sequences than CUs, rows longer than 57,344 tokens)
  p.spread = (a->K_max > 0 && p.draft != nullptr && (a->mode != nullptr || a->default_mode == SV_PLAIN) &&
              a->B <= 256 && (size_t)cfg.vocab > (size_t)57344)
                 ? 1
                 : 0;
  // other calls may run the sequence step in the row kernel (decided per
  // launch from its size)
  p.fuse = p.spread ? 0 : 1;
  return p;
}


// Enqueues the call in launches of at most kMaxSeqPerLaunch sequences and
// kMaxRowsPerLaunch rows; prof (or NULL) receives the stage events of the
// first launch.
hipError_t launch_call(sv::KParams p, int dtype, bool vec, hipStream_t s, hipEvent_t* prof) {
  size_t per = std::min(kMaxSeqPerLaunch, std::max<size_t>(1, kMaxRowsPerLaunch / p.R));
  // the draw-sum grid, nseq x D work-groups of kThreads, stays below 2^32 work-items
  if (p.spread) per = std::min(per, std::max<size_t>(1, kMaxRowsPerLaunch / (size_t)p.D));
  const int seq_per_launch = (int)per;
  hipError_t e = hipSuccess;
  for (int b0 = 0; b0 < p.B && e == hipSuccess; b0 += seq_per_launch) {
    p.b_base = b0;
    const int nseq = std::min(seq_per_launch, p.B - b0);
    p.b_end = b0 + nseq;
    e = sv::launch_verify(p, dtype, vec, nseq, s, b0 == 0 ? prof : nullptr);
  }
  return e;
}

}  // namespace

int spec_verify_run(sv_handle_t h, const sv_args* a, void* stream) {
  if (!h) return fail(SV_EINVAL, "handle is NULL");
  int rc = spec_verify_validate(&h->cfg, a);
  if (rc != SV_OK) return rc;
  if (a->B == 0) return SV_OK;
  const sv_config& cfg = h->cfg;
  Geometry g = geometry(&cfg);
  const sv::KParams p = make_params(cfg, g, h->ws, a);
  const bool vec = vector_loads(cfg, a);

  int prev = 0;
  if (hipGetDevice(&prev) != hipSuccess) return fail(SV_EHIP, "hipGetDevice failed");
  if (prev != cfg.device && hipSetDevice(cfg.device) != hipSuccess)
    return fail(SV_EHIP, "hipSetDevice failed");
  hipStream_t s = static_cast<hipStream_t>(stream);
  // Under stream capture the kernels become graph nodes; stage events are
  // left out.  No completion event is recorded per call: destroy and
  // profile_begin, which must wait for earlier runs, synchronise the device.
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cap) != hipSuccess) cap = hipStreamCaptureStatusNone;
  const bool capturing = cap != hipStreamCaptureStatusNone;
  hipEvent_t* ev = nullptr;
  if (!capturing && h->prof_next < h->prof_max) ev = &h->prof[4 * (size_t)h->prof_next++];
  const hipError_t e = launch_call(p, cfg.dtype, vec, s, ev);
  if (e == hipSuccess) h->has_run = true;
  if (prev != cfg.device) (void)hipSetDevice(prev);
  if (e != hipSuccess) return fail(SV_EHIP, std::string("launch failed: ") + hipGetErrorString(e));
  return SV_OK;
}

namespace {
void release_profile(sv_handle_t h) {
  for (hipEvent_t e : h->prof) (void)hipEventDestroy(e);
  h->prof.clear();
  h->prof_max = h->prof_next = 0;
}
}  // namespace

int spec_verify_profile_begin(sv_handle_t h, int max_calls) {
  if (!h) return fail(SV_EINVAL, "handle is NULL");
  if (max_calls < 1 || max_calls > 1000000) return fail(SV_EINVAL, "max_calls must be in [1, 10^6]");
  int prev = 0;
  if (hipGetDevice(&prev) != hipSuccess) return fail(SV_EHIP, "hipGetDevice failed");
  if (prev != h->cfg.device && hipSetDevice(h->cfg.device) != hipSuccess) return fail(SV_EHIP, "hipSetDevice failed");
  if (h->has_run) (void)hipDeviceSynchronize();  // earlier runs may still use the old events
  release_profile(h);
  hipError_t e = hipSuccess;
  for (int i = 0; i < 4 * max_calls && e == hipSuccess; ++i) {
    hipEvent_t ev;
    e = hipEventCreate(&ev);
    if (e == hipSuccess) h->prof.push_back(ev);
  }
  if (prev != h->cfg.device) (void)hipSetDevice(prev);
  if (e != hipSuccess) {
    release_profile(h);
    return fail(SV_EHIP, std::string("hipEventCreate failed: ") + hipGetErrorString(e));
  }
  h->prof_max = max_calls;
  h->prof_next = 0;
  return SV_OK;
}

int spec_verify_profile_end(sv_handle_t h, double* ms, int n_stages) {
  if (!h) return fail(SV_EINVAL, "handle is NULL");
  if (n_stages > 0 && !ms) return fail(SV_EINVAL, "ms is NULL");
  const int runs = h->prof_next;
  double sum[2] = {0.0, 0.0};
  hipError_t e = hipSuccess;
  if (runs > 0) e = hipEventSynchronize(h->prof[4 * (size_t)(runs - 1) + 3]);
  for (int i = 0; i < runs && e == hipSuccess; ++i) {
    float a = 0.0f, b = 0.0f;
    e = hipEventElapsedTime(&a, h->prof[4 * (size_t)i], h->prof[4 * (size_t)i + 1]);
    if (e == hipSuccess) e = hipEventElapsedTime(&b, h->prof[4 * (size_t)i + 2], h->prof[4 * (size_t)i + 3]);
    sum[0] += a;
    sum[1] += b;
  }
  release_profile(h);
  if (e != hipSuccess) return fail(SV_EHIP, std::string("reading the stage events failed: ") + hipGetErrorString(e));
  for (int i = 0; i < n_stages && i < 2; ++i) ms[i] = sum[i];
  return runs;
}

int spec_verify_stream_probe(const void* data, size_t bytes, void* out, void* stream) {
  if (!data || !out) return fail(SV_EINVAL, "stream probe: data and out must be device pointers");
  if (reinterpret_cast<uintptr_t>(data) % 16 != 0) return fail(SV_EINVAL, "stream probe: data must be 16-byte aligned");
  const hipError_t e = sv::launch_stream_probe(data, bytes, static_cast<uint32_t*>(out), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SV_EHIP, std::string("stream probe launch failed: ") + hipGetErrorString(e));
  return SV_OK;
}

int spec_verify_philox_words(uint64_t seed, const uint64_t* g, const uint32_t* t, const uint32_t* purpose,
                             int64_t n, uint32_t* out, void* stream) {
  if (n < 0) return fail(SV_EINVAL, "philox words: n must be >= 0");
  if (n == 0) return SV_OK;
  if (!g || !t || !purpose || !out) return fail(SV_EINVAL, "philox words: g, t, purpose and out must be device pointers");
  const hipError_t e = sv::launch_philox_words(seed, g, t, purpose, n, out, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SV_EHIP, std::string("philox words launch failed: ") + hipGetErrorString(e));
  return SV_OK;
}

int spec_verify_stream_probe_sweep(const void* data, size_t bytes, int loads_per_lane, int waves_per_cu, void* out,
                                   void* stream) {
  if (!data || !out) return fail(SV_EINVAL, "stream probe sweep: data and out must be device pointers");
  if (reinterpret_cast<uintptr_t>(data) % 16 != 0)
    return fail(SV_EINVAL, "stream probe sweep: data must be 16-byte aligned");
  if (loads_per_lane != 4 && loads_per_lane != 8 && loads_per_lane != 16)
    return fail(SV_EINVAL, "stream probe sweep: loads_per_lane must be 4, 8 or 16");
  if (waves_per_cu < 1 || waves_per_cu > 32)
    return fail(SV_EINVAL, "stream probe sweep: waves_per_cu must be in [1, 32]");
  const hipError_t e = sv::launch_stream_sweep(data, bytes, loads_per_lane, waves_per_cu, static_cast<uint32_t*>(out),
                                               static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SV_EHIP, std::string("stream probe sweep launch failed: ") + hipGetErrorString(e));
  return SV_OK;
}

int spec_verify_destroy(sv_handle_t h) {
  if (!h) return SV_OK;
  int prev = 0;
  (void)hipGetDevice(&prev);
  (void)hipSetDevice(h->cfg.device);
  hipError_t e = hipSuccess;
  if (h->has_run) e = hipDeviceSynchronize();
  release_profile(h);
  (void)hipFree(h->ws);
  (void)hipSetDevice(prev);
  delete h;
  if (e != hipSuccess) return fail(SV_EHIP, std::string("synchronising before the free failed: ") + hipGetErrorString(e));
  return SV_OK;
}

}  // extern "C"

// ------------------------------------------------------------------------
// The entry point that allocates nothing.  Its workspace is `scratch`, a
// file-scope device array that the runtime places once on every device this
// library's code runs on and keeps until the process ends.  In host code
// `scratch` only names the variable: its device address on the current
// device comes from hipGetSymbolAddress, taken once per device and kept in
// g_scratch_ptr, and only that address is passed to the kernels.
static_assert(SV_STATIC_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) unsigned char scratch[SV_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device `dev`.
hipError_t scratch_address(int dev, void** out) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}
}  // namespace

extern "C" int spec_verify_run_static(const sv_config* cfg, const sv_args* a, void* stream) {
  int rc = spec_verify_validate(cfg, a);
  if (rc != SV_OK) return rc;
  if (a->B == 0) return SV_OK;
  if (cfg->device >= kMaxDevices) return fail(SV_EINVAL, "device ordinal beyond the static scratch table (64)");
  // the workspace this call needs, laid out for its own B and K_max
  sv_config need = *cfg;
  need.max_batch = a->B;
  need.max_k = a->K_max;
  const Geometry g = geometry(&need);
  if (g.total > SV_STATIC_SCRATCH_BYTES)
    return fail(SV_ECAPACITY, "the call needs " + std::to_string(g.total) +
                                  " bytes of workspace, more than the static scratch buffer's " +
                                  std::to_string((unsigned long long)SV_STATIC_SCRATCH_BYTES));
  int prev = 0;
  if (hipGetDevice(&prev) != hipSuccess) return fail(SV_EHIP, "hipGetDevice failed");
  if (prev != cfg->device && hipSetDevice(cfg->device) != hipSuccess) return fail(SV_EHIP, "hipSetDevice failed");
  void* ws = nullptr;
  hipError_t e = scratch_address(cfg->device, &ws);
  if (e == hipSuccess) e = launch_call(make_params(need, g, ws, a), cfg->dtype, vector_loads(*cfg, a),
                                       static_cast<hipStream_t>(stream), nullptr);
  if (prev != cfg->device) (void)hipSetDevice(prev);
  if (e != hipSuccess) return fail(SV_EHIP, std::string("static run failed: ") + hipGetErrorString(e));
  return SV_OK;
}
