// The C ABI (include/sdm.h): argument checks, refusals, workspace layout and kernel launches.
//
// Refusal policy (sparse-delta-memory CHANGELOG.md 2.0.0, "Behavior changes" and "Known limitations"): float16
// raises; out-of-range settings (for example more writes or reads than slots) raise instead of being capped; a bank
// with fewer rows than slots raises instead of being read out of bounds; head_dim above 2^20 raises; there is no
// fallback path (only gfx950 runs); every refusal happens before any device work; the device check runs once per
// device (memoized), the argument checks on every call.
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "bwd_shape.h"
#include "layer.h"
#include "sdm_internal.h"

using namespace sdm;

namespace {

thread_local std::string g_err;

sdm_status fail(sdm_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
sdm_status fail(sdm_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

sdm_status ok() {
  g_err.clear();
  return SDM_OK;
}

size_t esize(int dt) { return dt == SDM_BF16 ? 2 : 4; }

// Number of position tuples with p_f < kp[f] and prod(p_f + 1) <= k (same enumeration as cand_table_kernel).
long long count_candidates(const int* kp, int F, int k) {
  int p[MAX_F] = {0, 0, 0, 0};
  long long c = 0;
  while (true) {
    long long prod = 1;
    for (int f = 0; f < F; ++f) prod *= p[f] + 1;
    if (prod <= k) ++c;
    int f = F - 1;
    for (; f >= 0; --f) {
      ++p[f];
      long long pp = 1;
      for (int g = 0; g <= f; ++g) pp *= p[g] + 1;
      if (p[f] < kp[f] && pp <= k) break;
      p[f] = 0;
    }
    if (f < 0) break;
  }
  return c;
}

sdm_status make_plan(const Dims& D, int k, const char* what, TopkPlan* P) {
  if (k < 1 || (long long)k > D.N || k > MAX_K)
    return fail(SDM_ERR_RANGE, "%s = %d out of range [1, min(N = %lld, %d)]", what, k, D.N, MAX_K);
  P->k = k;
  P->kpmax = 0;
  int nfmax = 0;
  for (int f = 0; f < MAX_F; ++f) P->kp[f] = 0;
  for (int f = 0; f < D.F; ++f) {
    P->kp[f] = k < D.widths[f] ? k : D.widths[f];
    if (P->kp[f] > P->kpmax) P->kpmax = P->kp[f];
    if (D.widths[f] > nfmax) nfmax = D.widths[f];
  }
  const long long nc = count_candidates(P->kp, D.F, k);
  if (nc > MAX_CAND)
    return fail(SDM_ERR_RANGE, "%s = %d with these factor widths gives %lld candidate tuples (limit %d)", what, k,
                nc, MAX_CAND);
  P->ncand = (int)nc;
  P->cand_pow2 = pow2_ceil((int)nc);
  P->nf_pow2 = pow2_ceil(nfmax);
  return SDM_OK;
}

// The chunk the kernels run for a requested chunk_size: the chunk_size itself when it fits their limits (at most
// MAX_CHUNK tokens and MAX_CHUNK_EVENTS write events), else its largest divisor that does. The chunk size changes
// results only through rounding (CHANGELOG 2.0.0, "Upgrading from v1"), so equal sub-chunks give a result of the
// requested chunk size; chunk boundaries still fall on every multiple of chunk_size, so calls split there give the
// bits of one call.
int kernel_chunk(int C, int W) {
  for (int c = C; c >= 1; --c)
    if (C % c == 0 && c <= MAX_CHUNK && (long long)c * W <= MAX_CHUNK_EVENTS) return c;
  return 1;
}

// op: SDM_OP_TOPK (k given), SDM_OP_WRITE_READ, SDM_OP_DECODE, SDM_OP_BACKWARD (the write/read's config),
// SDM_OP_DECODE_STEPS (tokens = the number of steps)
sdm_status validate(const sdm_config* cfg, int op, int k, Dims* D, TopkPlan* pw, TopkPlan* pr) {
  if (!cfg) return fail(SDM_ERR_NULL, "cfg is NULL");
  if (op < SDM_OP_TOPK || op > SDM_OP_DECODE_STEPS) return fail(SDM_ERR_RANGE, "unknown op %d", op);
  const bool chunked = op == SDM_OP_WRITE_READ || op == SDM_OP_BACKWARD;
  const int act = cfg->act_dtype, bank = cfg->bank_dtype;
  if (act == SDM_F16 || (op != SDM_OP_TOPK && bank == SDM_F16))
    return fail(SDM_ERR_DTYPE, "float16 is not supported (use float32 or bfloat16)");
  if (act != SDM_F32 && act != SDM_BF16) return fail(SDM_ERR_DTYPE, "unknown act_dtype %d", act);
  if (op != SDM_OP_TOPK && bank != SDM_F32 && bank != SDM_BF16) return fail(SDM_ERR_DTYPE, "unknown bank_dtype %d", bank);
  if (cfg->batch < 0 || cfg->tokens < 0 || cfg->heads < 0)
    return fail(SDM_ERR_RANGE, "batch, tokens and heads must be >= 0");
  if (op == SDM_OP_DECODE && cfg->tokens != 1)
    return fail(SDM_ERR_RANGE, "sdm_decode_step takes exactly one token per stream (tokens = %d)", cfg->tokens);
  if ((long long)cfg->batch * cfg->heads > 65535 && chunked)
    return fail(SDM_ERR_RANGE, "batch * heads = %lld exceeds 65535 streams", (long long)cfg->batch * cfg->heads);
  if ((long long)cfg->batch * cfg->heads > 0x7FFFFFFFLL)
    return fail(SDM_ERR_RANGE, "batch * heads exceeds 2^31 - 1");
  if ((long long)cfg->batch * cfg->tokens * cfg->heads > (1LL << 24))
    return fail(SDM_ERR_RANGE, "batch * tokens * heads exceeds 2^24 token rows per call");
  const int F = cfg->num_factors;
  if (F < 1 || F > MAX_F) return fail(SDM_ERR_RANGE, "num_factors = %d out of range [1, %d]", F, MAX_F);
  memset(D, 0, sizeof *D);
  long long N = 1;
  for (int f = 0; f < F; ++f) {
    const int n = cfg->factor_widths[f];
    if (n < 1 || n > MAX_NF) return fail(SDM_ERR_RANGE, "factor_widths[%d] = %d out of range [1, %d]", f, n, MAX_NF);
    D->widths[f] = n;
    N *= n;
    if (N > 0x7FFFFFFFLL) return fail(SDM_ERR_RANGE, "slot count (product of factor widths) exceeds 2^31 - 1");
  }
  if (cfg->subkey_dim < 1 || (long long)F * cfg->subkey_dim > MAX_FDK)
    return fail(SDM_ERR_RANGE, "subkey_dim = %d out of range (num_factors * subkey_dim must be in [1, %d])",
                cfg->subkey_dim, MAX_FDK);
  D->B = cfg->batch; D->T = cfg->tokens; D->H = cfg->heads; D->F = F; D->dk = cfg->subkey_dim;
  D->act = act; D->bank = bank; D->N = N; D->S = cfg->batch * cfg->heads;
  if (cfg->topk_scoring < SDM_SCORING_AUTO || cfg->topk_scoring > SDM_SCORING_FILTERED)
    return fail(SDM_ERR_RANGE, "topk_scoring = %d (0 auto, 1 direct, 2 filtered)", cfg->topk_scoring);
  D->scoring = cfg->topk_scoring;
  if (op == SDM_OP_TOPK) return make_plan(*D, k, "k", pw);
  if (cfg->shared_bank != 0 && cfg->shared_bank != 1)
    return fail(SDM_ERR_RANGE, "shared_bank = %d must be 0 or 1", cfg->shared_bank);
  if (cfg->shared_bank && op != SDM_OP_WRITE_READ)
    return fail(SDM_ERR_RANGE, "shared_bank applies to sdm_write_read only (a decode step's streams own their banks)");
  D->shared = cfg->shared_bank;

  const int d = cfg->head_dim;
  if (d < 1 || d > (1 << 20)) return fail(SDM_ERR_RANGE, "head_dim = %d out of range [1, 2^20]", d);
  const int lane = bank == SDM_BF16 ? 8 : 4;
  if (d % lane) return fail(SDM_ERR_LAYOUT, "head_dim = %d must be a multiple of %d for this bank dtype", d, lane);
  D->d = d;
  D->W = cfg->num_writes; D->R = cfg->num_reads;
  sdm_status s = make_plan(*D, D->W, "num_writes", pw);
  if (s != SDM_OK) return s;
  s = make_plan(*D, D->R, "num_reads", pr);
  if (s != SDM_OK) return s;
  if (cfg->bank_rows < N)
    return fail(SDM_ERR_BANK_TOO_SMALL, "bank_rows = %lld is smaller than the slot count N = %lld",
                (long long)cfg->bank_rows, N);
  D->rows = cfg->bank_rows;
  const long long ld = cfg->bank_row_stride ? cfg->bank_row_stride : d;
  if (ld < d || (ld * (bank == SDM_BF16 ? 2 : 4)) % 16 != 0)
    return fail(SDM_ERR_LAYOUT, "bank_row_stride = %lld must be >= head_dim = %d and a multiple of 16 bytes", ld, d);
  D->ld = ld;
  if (op == SDM_OP_BACKWARD && (long long)D->S * D->T * D->W >= (1LL << 31))
    return fail(SDM_ERR_RANGE, "the backward snapshot would hold batch * heads * tokens * num_writes = %lld rows "
                "(2^31 or more)", (long long)D->S * D->T * D->W);
  if (chunked) {
    const int C = cfg->chunk_size;
    if (C < 1 || C > MAX_CHUNK_SIZE)
      return fail(SDM_ERR_RANGE, "chunk_size = %d out of range [1, %d]", C, MAX_CHUNK_SIZE);
    D->C = kernel_chunk(C, D->W);
    D->nch = (D->T + D->C - 1) / D->C;
  } else {
    D->C = 1;
    D->nch = 1;
  }
  return SDM_OK;
}

// Device check, memoized per device: 0 unknown, 1 gfx950, 2 other.
std::atomic<int> g_dev_ok[64];
size_t g_dev_lds[64];

sdm_status check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(SDM_ERR_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= 64) return fail(SDM_ERR_DEVICE, "device index %d not supported", dev);
  int st = g_dev_ok[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) != hipSuccess) return fail(SDM_ERR_HIP, "hipGetDeviceProperties failed");
    st = strncmp(p.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_dev_lds[dev] = p.sharedMemPerBlock;
    g_dev_ok[dev].store(st, std::memory_order_release);
  }
  if (st != 1) return fail(SDM_ERR_DEVICE, "device %d is not gfx950 (MI355X); no other GPU is supported", dev);
  return SDM_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

WsLayout layout(const Dims& D, int op) {
  WsLayout L;
  memset(&L, 0, sizeof L);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t r = o;
    o = align256(o + bytes);
    return r;
  };
  L.cand = take(2 * MAX_CAND * 8);
  L.snorm = take((size_t)D.H * D.F * 4);
  if (op == SDM_OP_DECODE || op == SDM_OP_DECODE_STEPS) {  // ids and weights (steps: ids and scores) per token
    const size_t nw = (size_t)D.S * D.T * D.W, nr = (size_t)D.S * D.T * D.R;
    L.widx = take(nw * 4);
    L.wwt = take(nw * 4);
    L.ridx = take(nr * 4);
    L.rwt = take(nr * 4);
  }
  if (op == SDM_OP_WRITE_READ) {
    const size_t nw = (size_t)D.S * D.T * D.W, nr = (size_t)D.S * D.T * D.R;
    const size_t nc = (size_t)D.S * D.nch;
    L.widx = take(nw * 4);
    L.wwt = take(nw * 4);
    L.ridx = take(nr * 4);
    L.rwt = take(nr * 4);
    L.chunks = take(nc * (size_t)chunk_layout(D.C, D.W, D.R).bytes);
    L.counts = take(nc * sizeof(ChunkCounts));
    if (D.shared) {
      L.owner = take((size_t)D.H * (size_t)D.N * 4);
      L.conflict = take(4);
    }
  }
  if (op == SDM_OP_BACKWARD) {
    const size_t nw = (size_t)D.S * D.T * D.W, nr = (size_t)D.S * D.T * D.R;
    long long sumn = 0;
    for (int f = 0; f < D.F; ++f) sumn += D.widths[f];
    L.widx = take(nw * 4);
    L.wwt = take(nw * 4);
    L.ridx = take(nr * 4);
    L.rwt = take(nr * 4);
    L.part = take((size_t)bwd_nsl(D) * D.S * D.T * (D.W + D.R + 2) * 4);
    L.ds = take((size_t)D.S * D.T * (D.W + D.R) * 4);
    L.sgpart = take((size_t)bwd_row_blocks(D) * D.H * sumn * D.dk * 4);
    L.mrho = take(nw * 4);
    L.mread = take(nr * 4);
    const int G = bwd_group_tokens(D);
    if (G > 1) {
      const size_t st = (size_t)D.S * D.T, nb = (size_t)D.S * ((D.T + G - 1) / G);
      L.gent = take(st * 4);
      L.gcnt = take(nb * 4);
      L.giter = take(st * 4);
      L.gn = take((size_t)D.S * 4);
    }
  }
  L.total = o;
  return L;
}

struct Range {
  const void* p;
  size_t n;
  const char* name;
};

bool overlap(const Range& a, const Range& b) {
  if (!a.p || !b.p || a.n == 0 || b.n == 0) return false;
  const uintptr_t a0 = (uintptr_t)a.p, a1 = a0 + a.n, b0 = (uintptr_t)b.p, b1 = b0 + b.n;
  return a0 < b1 && b0 < a1;
}

// Every output must be disjoint from every other range (inputs and outputs).
sdm_status check_alias(const Range* outs, int nout, const Range* ins, int nin) {
  for (int i = 0; i < nout; ++i) {
    for (int j = 0; j < nin; ++j)
      if (overlap(outs[i], ins[j])) return fail(SDM_ERR_ALIAS, "%s overlaps %s", outs[i].name, ins[j].name);
    for (int j = i + 1; j < nout; ++j)
      if (overlap(outs[i], outs[j])) return fail(SDM_ERR_ALIAS, "%s overlaps %s", outs[i].name, outs[j].name);
  }
  return SDM_OK;
}

sdm_status need(const void* p, const char* name) {
  return p ? SDM_OK : fail(SDM_ERR_NULL, "%s is NULL", name);
}

sdm_status aligned(const void* p, size_t a, const char* name) {
  return ((uintptr_t)p % a) == 0 ? SDM_OK : fail(SDM_ERR_LAYOUT, "%s must be %zu-byte aligned", name, a);
}

sdm_status check_ws(const void* ws, size_t ws_bytes, size_t need_bytes) {
  if (need_bytes == 0) return SDM_OK;
  if (!ws) return fail(SDM_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need_bytes);
  if ((uintptr_t)ws % 256) return fail(SDM_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < need_bytes) return fail(SDM_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, need_bytes);
  return SDM_OK;
}

// ------------------------------------------------------------------------------------------- kernel timing
struct ProfPair {
  int kernel;
  hipEvent_t a, b;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfPair> g_prof_pending;
std::vector<hipEvent_t> g_prof_pool;
double g_prof_ms[SDM_K_COUNT];
long long g_prof_n[SDM_K_COUNT];

hipEvent_t prof_event() {
  if (!g_prof_pool.empty()) {
    hipEvent_t e = g_prof_pool.back();
    g_prof_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Runs `launch` (returns hipError_t); when timing is on, brackets it with events on stream st.
template <typename F>
hipError_t timed(int kernel, hipStream_t st, F&& launch) {
  bool on;
  {
    std::lock_guard<std::mutex> g(g_prof_mu);
    on = g_prof_on;
  }
  if (!on) return launch();
  ProfPair p;
  {
    std::lock_guard<std::mutex> g(g_prof_mu);
    p.kernel = kernel;
    p.a = prof_event();
    p.b = prof_event();
  }
  if (p.a) (void)hipEventRecord(p.a, st);
  const hipError_t e = launch();
  if (p.b) (void)hipEventRecord(p.b, st);
  std::lock_guard<std::mutex> g(g_prof_mu);
  if (p.a && p.b) g_prof_pending.push_back(p);
  return e;
}

sdm_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return SDM_OK;
  return fail(SDM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define TRY(x)                        \
  do {                                \
    sdm_status _s = (x);              \
    if (_s != SDM_OK) return _s;      \
  } while (0)

// The backward snapshot's element: the bank dtype (snapshot_dtype 0), or bfloat16 (SDM_BF16; the same as 0 on a
// bfloat16 bank) [CHANGELOG 2.0.0, "New": bf16 snapshots on a float32 bank]. A bfloat16 snapshot of a float32
// bank has native kernels when the held-row loop writes the snapshot and the fast reverse sweep (W, R <= 128) reads
// it; other training calls are refused before any work, as the pages refuse snapshot routes they lack.
sdm_status snapshot_kind(const sdm_config* cfg, const Dims& D, int* mode) {
  *mode = SNAP_BANK;
  const int sd = cfg->snapshot_dtype;
  if (sd == 0 || (sd == SDM_BF16 && D.bank == SDM_BF16)) return SDM_OK;
  if (sd != SDM_BF16 && sd != SDM_FP8 && sd != SDM_INT4)
    return fail(SDM_ERR_DTYPE, "snapshot_dtype = %d (0: the bank dtype, SDM_BF16, SDM_FP8 or SDM_INT4)", sd);
  const char* name = sd == SDM_BF16 ? "bfloat16" : sd == SDM_FP8 ? "fp8" : "int4";
  if (sd != SDM_BF16) {
    if (D.bank != SDM_F32)
      return fail(SDM_ERR_RANGE, "no native route for %s snapshots of a bfloat16 bank (only a float32 bank's snapshot "
                  "is quantized): use snapshot_dtype 0", name);
    // the pages' refusals for quantized snapshots (CHANGELOG 2.0.0, "Behavior changes")
    const int n = (D.d + 127) / 128;
    if (D.d > 16384 || D.d % 4 != 0 || D.d % n != 0 || (D.d / n) % 4 != 0)
      return fail(SDM_ERR_RANGE, "no quantized route for head_dim %d (above 16384, not a multiple of 4, or not "
                  "splitting into ceil(head_dim / 128) = %d equal column slices of 16-byte rows): use snapshot_dtype 0",
                  D.d, n);
    if (sd == SDM_INT4 && (D.d / n) % 8 == 4)
      return fail(SDM_ERR_RANGE, "no native route for int4 snapshots of a float32 bank whose %d column slices are %d "
                  "columns wide (4 mod 8): use SDM_FP8 or snapshot_dtype 0", n, D.d / n);
    // this library's quantization groups
    if (D.d % SNAP_GROUP != 0)
      return fail(SDM_ERR_RANGE, "no native route for %s snapshots with head_dim %d (groups of %d columns): use "
                  "snapshot_dtype 0", name, D.d, SNAP_GROUP);
  }
  if (!loop_held_snap_ok(D) || !bwd_fast(D))
    return fail(SDM_ERR_RANGE, "no native route for a %s snapshot of a float32 bank at these settings (it "
                "needs the held-row loop: chunk a power of two in [8, 128], at most 32 terms per lane group, and "
                "num_writes, num_reads <= 128): use snapshot_dtype 0", name);
  *mode = sd == SDM_BF16 ? SNAP_BF16 : sd == SDM_FP8 ? SNAP_FP8 : SNAP_INT4;
  return SDM_OK;
}

// The bank gradient's element (cfg.grad_bank_dtype): float32 (0), or bfloat16 (SDM_BF16: a bfloat16 bank; in the
// backward, the fast reverse sweep's shapes only).
sdm_status grad_bank_kind(const sdm_config* cfg, const Dims& D, bool backward, bool* bf16) {
  const int g = cfg->grad_bank_dtype;
  if (g != SDM_F32 && g != SDM_BF16)
    return fail(SDM_ERR_DTYPE, "grad_bank_dtype = %d (0: float32, SDM_BF16: the bank dtype of a bfloat16 bank)", g);
  *bf16 = g == SDM_BF16;
  if (!*bf16) return SDM_OK;
  if (D.bank != SDM_BF16)
    return fail(SDM_ERR_RANGE, "a bfloat16 bank gradient is the bank dtype of a bfloat16 bank; a float32 bank's "
                "gradient is float32 (grad_bank_dtype 0)");
  if (backward && !bwd_fast(D))
    return fail(SDM_ERR_RANGE, "no native route for a bfloat16 bank gradient with num_writes %d, num_reads %d (at "
                "most 128 each): use grad_bank_dtype 0", D.W, D.R);
  return SDM_OK;
}

// Bytes of the backward snapshot of mode `mode` (snapshot_kind) for D.
size_t snapshot_bytes(const Dims& D, int mode) {
  const size_t rows = (size_t)D.S * D.T * D.W;
  if (mode == SNAP_FP8 || mode == SNAP_INT4)
    return rows * (size_t)(snap_row_elem_bytes(mode, D.d) + snap_row_scale_bytes(D.d));
  return rows * (size_t)D.d * (mode == SNAP_BF16 ? 2 : esize(D.bank));
}

}  // namespace

extern "C" {

const char* sdm_last_error(void) { return g_err.c_str(); }

sdm_status sdm_workspace_size(const sdm_config* cfg, int32_t op, int32_t k, size_t* bytes) {
  if (!bytes) return fail(SDM_ERR_NULL, "bytes is NULL");
  Dims D;
  TopkPlan pw, pr;
  TRY(validate(cfg, op, k, &D, &pw, &pr));
  *bytes = layout(D, op).total;
  return ok();
}

sdm_status topk_product_keys(const sdm_config* cfg, const void* queries, const void* subkeys, int32_t k,
                             int32_t* idx, float* scores, void* workspace, size_t workspace_bytes, void* stream) {
  Dims D;
  TopkPlan P, unused;
  TRY(validate(cfg, SDM_OP_TOPK, k, &D, &P, &unused));
  const long long rows = (long long)D.B * D.T * D.H;
  long long sumn = 0;
  for (int f = 0; f < D.F; ++f) sumn += D.widths[f];
  const size_t ea = esize(D.act);
  if (rows > 0) {
    TRY(need(queries, "queries"));
    TRY(need(idx, "idx"));
  }
  if (D.H > 0) TRY(need(subkeys, "subkeys"));
  const WsLayout L = layout(D, SDM_OP_TOPK);
  TRY(check_ws(workspace, workspace_bytes, L.total));
  const Range ins[] = {{queries, (size_t)rows * D.F * D.dk * ea, "queries"},
                       {subkeys, (size_t)D.H * sumn * D.dk * ea, "subkeys"}};
  const Range outs[] = {{idx, (size_t)rows * k * 4, "idx"},
                        {scores, (size_t)rows * k * 4, "scores"},
                        {workspace, L.total, "workspace"}};
  TRY(check_alias(outs, 3, ins, 2));
  TRY(check_device());
  if (rows == 0) return ok();
  hipStream_t st = (hipStream_t)stream;
  unsigned char* ws = (unsigned char*)workspace;
  TRY(hip_status(timed(SDM_K_CAND, st, [&] { return launch_cand_tables(&P, 1, D.F, (uint64_t*)(ws + L.cand), st); }),
                 "candidate table launch"));
  TopkArgs a;
  memset(&a, 0, sizeof a);
  a.queries[0] = queries;
  a.subkeys = subkeys;
  a.cand[0] = (const uint64_t*)(ws + L.cand);
  a.plan[0] = P;
  a.nkinds = 1;
  a.stream_major = 0;
  a.ids[0] = idx;
  a.vals[0] = scores;
  a.snorm = (float*)(ws + L.snorm);
  TRY(hip_status(timed(SDM_K_TOPK, st, [&] { return launch_topk(D, a, st); }), "top-k launch"));
  return ok();
}

// The write/read; with a snapshot (not NULL) also the backward's snapshot, through the segmented chunk loop.
// The pipelined write/read: when the chunk loop's workgroups (one per stream and column slice) leave at least half of
// the compute units free, the sequence runs as up to PIPE_MAX pieces of whole chunks, and the top-k and chunk plan
// of piece p + 1 (bank-independent) run on a side stream beside the chunk loop of piece p on the caller's stream.
// The loop of piece p waits for its own plan only, and its launches are those of calls split at the pieces'
// chunk boundaries, which give the bits of one call. With the chip full of loop workgroups the side stream's work
// would only queue behind them, so it is not used then. The side stream (default priority) and its events are made
// once per device and kept until the process ends; a call forks the side stream from the caller's stream and joins
// it back before it returns. A call on a capturing stream runs in order on that stream: a side stream that joined a
// capture would stay in it until the capture ends, and another thread's calls would then be recorded into it.
namespace {
constexpr int PIPE_MAX = 16;
struct PipeDev {
  hipStream_t side = nullptr;
  hipEvent_t ev[PIPE_MAX + 2] = {};  // ev[p]: piece p planned; ev[PIPE_MAX]: fork; ev[PIPE_MAX + 1]: join
  int cus = 0;
  bool tried = false;
};
constexpr int PIPE_DEVICES = 64;
std::mutex g_pipe_mu;  // held while a call enqueues its pieces (one set of events per device)
PipeDev g_pipe[PIPE_DEVICES];

// The current device's side stream and events for a call on `st`, or nullptr: `st` is capturing, or they could not
// be made (another thread's capture may forbid it for now; then a later call tries again).
static PipeDev* pipe_device(hipStream_t st) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= PIPE_DEVICES) return nullptr;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return nullptr;
  PipeDev& p = g_pipe[dev];
  if (!p.tried) {
    PipeDev n;
    bool made = hipDeviceGetAttribute(&n.cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
                hipStreamCreateWithFlags(&n.side, hipStreamNonBlocking) == hipSuccess;
    int ne = 0;
    while (made && ne < PIPE_MAX + 2) {
      made = hipEventCreateWithFlags(&n.ev[ne], hipEventDisableTiming) == hipSuccess;
      if (made) ++ne;
    }
    if (!made) {  // give back what was made
      for (int i = 0; i < ne; ++i) (void)hipEventDestroy(n.ev[i]);
      if (n.side) (void)hipStreamDestroy(n.side);
      (void)hipGetLastError();
      return nullptr;
    }
    n.tried = true;
    p = n;
  }
  return &p;
}

// Chunks per piece of a pipelined call, or 0 to run the call in order on the caller's stream.
static int pipe_chunks(const Dims& D, bool snapshot, const PipeDev* pd) {
  if (pd == nullptr || D.shared || D.nch < 2) return 0;
  if (loop_workgroups(D, snapshot) * 2 > pd->cus) return 0;
  const int per = (D.nch + PIPE_MAX - 1) / PIPE_MAX;
  // a window of several batch rows is a multiple of 16 tokens (the top-k's rows of a wave stay in one batch row)
  if (D.B > 1 && ((per * D.C) % 16 != 0 || D.T % 16 != 0)) return 0;
  return per;
}
}  // namespace

static sdm_status write_read_impl(const sdm_config* cfg, const void* write_keys, const void* read_queries,
                           const void* values, const void* forget_gate, const void* input_gate, const void* subkeys,
                           void* bank, void* out, void* snapshot, int32_t* write_idx, int32_t* read_idx,
                           void* workspace, size_t workspace_bytes, void* stream) {
  Dims D;
  TopkPlan pw, pr;
  TRY(validate(cfg, SDM_OP_WRITE_READ, 0, &D, &pw, &pr));
  int snap_mode = SNAP_BANK;
  if (snapshot) TRY(snapshot_kind(cfg, D, &snap_mode));
  const size_t snap_bytes = snapshot_bytes(D, snap_mode);
  if (snapshot || cfg->shared_bank) {
    if (cfg->shared_bank && snapshot)
      return fail(SDM_ERR_RANGE, "a shared bank has no backward (sdm_write_read_save refuses shared_bank)");
    if (snapshot && (long long)D.S * D.T * D.W >= (1LL << 31))
      return fail(SDM_ERR_RANGE, "the backward snapshot would hold batch * heads * tokens * num_writes = %lld rows "
                  "(2^31 or more)", (long long)D.S * D.T * D.W);
  }
  const long long rows = (long long)D.B * D.T * D.H;
  long long sumn = 0;
  for (int f = 0; f < D.F; ++f) sumn += D.widths[f];
  const size_t ea = esize(D.act), eb = esize(D.bank);
  const size_t bank_bytes = (size_t)(D.shared ? D.H : D.S) * (size_t)D.rows * (size_t)D.ld * eb;
  if (rows > 0) {
    TRY(need(write_keys, "write_keys"));
    TRY(need(read_queries, "read_queries"));
    TRY(need(values, "values"));
    TRY(need(forget_gate, "forget_gate"));
    TRY(need(input_gate, "input_gate"));
    TRY(need(subkeys, "subkeys"));
    TRY(need(bank, "bank"));
    TRY(need(out, "out"));
  }
  TRY(aligned(bank, 16, "bank"));
  if (snapshot) TRY(aligned(snapshot, 16, "snapshot"));
  const WsLayout L = layout(D, SDM_OP_WRITE_READ);
  TRY(check_ws(workspace, workspace_bytes, L.total));
  const size_t qb = (size_t)rows * D.F * D.dk * ea;
  const Range ins[] = {{write_keys, qb, "write_keys"},
                       {read_queries, qb, "read_queries"},
                       {values, (size_t)rows * D.d * ea, "values"},
                       {forget_gate, (size_t)rows * ea, "forget_gate"},
                       {input_gate, (size_t)rows * ea, "input_gate"},
                       {subkeys, (size_t)D.H * sumn * D.dk * ea, "subkeys"}};
  const Range outs[] = {{bank, bank_bytes, "bank"},
                        {out, (size_t)rows * D.d * ea, "out"},
                        {write_idx, (size_t)rows * D.W * 4, "write_idx"},
                        {read_idx, (size_t)rows * D.R * 4, "read_idx"},
                        {workspace, L.total, "workspace"},
                        {snapshot, snap_bytes, "snapshot"}};
  TRY(check_alias(outs, 6, ins, 6));
  TRY(check_device());
  if (rows == 0) return ok();
  hipStream_t st = (hipStream_t)stream;
  unsigned char* ws = (unsigned char*)workspace;
  const TopkPlan plans[2] = {pw, pr};
  TopkArgs ta;
  memset(&ta, 0, sizeof ta);
  ta.queries[0] = write_keys;
  ta.queries[1] = read_queries;
  ta.subkeys = subkeys;
  ta.cand[0] = (const uint64_t*)(ws + L.cand);
  ta.cand[1] = (const uint64_t*)(ws + L.cand) + MAX_CAND;
  ta.plan[0] = pw;
  ta.plan[1] = pr;
  ta.nkinds = 2;
  ta.stream_major = 1;
  ta.ids[0] = (int32_t*)(ws + L.widx);
  ta.ids[1] = (int32_t*)(ws + L.ridx);
  ta.vals[0] = (float*)(ws + L.wwt);
  ta.vals[1] = (float*)(ws + L.rwt);
  ta.user_ids[0] = write_idx;
  ta.user_ids[1] = read_idx;
  ta.snorm = (float*)(ws + L.snorm);
  const int32_t* abort = D.shared ? (const int32_t*)(ws + L.conflict) : nullptr;
  PlanArgs pa;
  pa.abort = abort;
  pa.widx = (const int32_t*)(ws + L.widx);
  pa.wwt = (const float*)(ws + L.wwt);
  pa.ridx = (const int32_t*)(ws + L.ridx);
  pa.rwt = (const float*)(ws + L.rwt);
  pa.alpha = forget_gate;
  pa.beta = input_gate;
  pa.chunks = ws + L.chunks;
  pa.counts = (ChunkCounts*)(ws + L.counts);
  // the loop that runs: held-row (also with a snapshot), narrow (not with a snapshot) or segmented; only the
  // segmented loop reads the slot segments, only the narrow one lane-major terms
  const bool held = snapshot ? loop_held_snap_ok(D) : loop_held_path(D);
  const bool narrow = !held && !snapshot && loop_narrow_path(D);
  pa.scat = held || narrow ? 0 : 1;
  pa.lanemajor = narrow && loop_narrow_lanemajor(D) ? 1 : 0;
  pa.evcode = snapshot ? 1 : 0;
  LoopArgs la;
  la.alpha = forget_gate;
  la.beta = input_gate;
  la.values = values;
  la.chunks = pa.chunks;
  la.counts = pa.counts;
  la.bank = bank;
  la.out = out;
  la.abort = abort;
  la.snap = snapshot;
  la.snap_mode = snap_mode;
  std::unique_lock<std::mutex> lock(g_pipe_mu);
  PipeDev* pd = pipe_device(st);
  const int per = pipe_chunks(D, snapshot != nullptr, pd);
  if (per == 0) {  // in order on the caller's stream
    lock.unlock();
    TRY(hip_status(timed(SDM_K_CAND, st, [&] { return launch_cand_tables(plans, 2, D.F, (uint64_t*)(ws + L.cand), st); }),
                   "candidate table launch"));
    TRY(hip_status(timed(SDM_K_TOPK, st, [&] { return launch_topk(D, ta, st); }), "top-k launch"));
    if (D.shared)  // the streams of a head must address disjoint slots; if not, the plan and the loop do nothing
      TRY(hip_status(launch_shared_check(D, (const int32_t*)(ws + L.widx), (const int32_t*)(ws + L.ridx),
                                         (int32_t*)(ws + L.owner), (int32_t*)(ws + L.conflict), st),
                     "shared-bank check launch"));
    TRY(hip_status(timed(SDM_K_PLAN, st, [&] { return launch_plan(D, pa, st); }), "chunk plan launch"));
    TRY(hip_status(timed(SDM_K_LOOP, st, [&] { return launch_loop(D, la, st); }), "chunk loop launch"));
    return ok();
  }
  // pipelined: fork the side stream from the caller's stream, then per piece the top-k and plan on the side stream
  // and the loop on the caller's stream after that piece's plan; the side stream is joined back on every exit
  hipStream_t side = pd->side;
  TRY(hip_status(hipEventRecord(pd->ev[PIPE_MAX], st), "fork event record"));
  TRY(hip_status(hipStreamWaitEvent(side, pd->ev[PIPE_MAX], 0), "fork event wait"));
  auto pieces = [&]() -> sdm_status {
    TRY(hip_status(timed(SDM_K_CAND, side, [&] {
      return launch_cand_tables(plans, 2, D.F, (uint64_t*)(ws + L.cand), side); }), "candidate table launch"));
    for (int c0 = 0, p = 0; c0 < D.nch; c0 += per, ++p) {
      const int nc = D.nch - c0 < per ? D.nch - c0 : per;
      ta.t0 = c0 * D.C;
      ta.tn = ((c0 + nc) * D.C < D.T ? (c0 + nc) * D.C : D.T) - ta.t0;
      TRY(hip_status(timed(SDM_K_TOPK, side, [&] { return launch_topk(D, ta, side); }), "top-k launch"));
      pa.ch0 = c0;
      pa.chn = nc;
      TRY(hip_status(timed(SDM_K_PLAN, side, [&] { return launch_plan(D, pa, side); }), "chunk plan launch"));
      TRY(hip_status(hipEventRecord(pd->ev[p], side), "piece event record"));
      TRY(hip_status(hipStreamWaitEvent(st, pd->ev[p], 0), "piece event wait"));
      la.ch0 = c0;
      la.ch1 = c0 + nc;
      TRY(hip_status(timed(SDM_K_LOOP, st, [&] { return launch_loop(D, la, st); }), "chunk loop launch"));
    }
    return ok();
  };
  const sdm_status rc = pieces();
  hipError_t ej = hipEventRecord(pd->ev[PIPE_MAX + 1], side);
  if (ej == hipSuccess) ej = hipStreamWaitEvent(st, pd->ev[PIPE_MAX + 1], 0);
  if (rc != SDM_OK) return rc;
  TRY(hip_status(ej, "join event"));
  return ok();
}


sdm_status sdm_write_read(const sdm_config* cfg, const void* write_keys, const void* read_queries,
                          const void* values, const void* forget_gate, const void* input_gate, const void* subkeys,
                          void* bank, void* out, int32_t* write_idx, int32_t* read_idx, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return write_read_impl(cfg, write_keys, read_queries, values, forget_gate, input_gate, subkeys, bank, out, nullptr,
                         write_idx, read_idx, workspace, workspace_bytes, stream);
}

sdm_status sdm_write_read_save(const sdm_config* cfg, const void* write_keys, const void* read_queries,
                               const void* values, const void* forget_gate, const void* input_gate,
                               const void* subkeys, void* bank, void* out, void* snapshot, int32_t* write_idx,
                               int32_t* read_idx, void* workspace, size_t workspace_bytes, void* stream) {
  if (cfg && (long long)cfg->batch * cfg->tokens * cfg->heads > 0 && !snapshot)
    return fail(SDM_ERR_NULL, "snapshot is NULL");
  if (cfg && cfg->shared_bank)
    return fail(SDM_ERR_RANGE, "a shared bank has no backward (sdm_write_read_save refuses shared_bank)");
  return write_read_impl(cfg, write_keys, read_queries, values, forget_gate, input_gate, subkeys, bank, out,
                         snapshot, write_idx, read_idx, workspace, workspace_bytes, stream);
}

sdm_status sdm_write_read_backward(const sdm_config* cfg, const void* write_keys, const void* read_queries,
                                   const void* values, const void* forget_gate, const void* input_gate,
                                   const void* subkeys, void* bank, const void* snapshot, const void* grad_out,
                                   void* grad_bank, float* grad_write_keys, float* grad_read_queries,
                                   float* grad_values, float* grad_forget_gate, float* grad_input_gate,
                                   float* grad_subkeys, void* workspace, size_t workspace_bytes, void* stream) {
  Dims D;
  TopkPlan pw, pr;
  TRY(validate(cfg, SDM_OP_BACKWARD, 0, &D, &pw, &pr));
  int snap_mode = SNAP_BANK;
  TRY(snapshot_kind(cfg, D, &snap_mode));
  bool gb16 = false;
  TRY(grad_bank_kind(cfg, D, true, &gb16));
  const long long rows = (long long)D.B * D.T * D.H;
  long long sumn = 0;
  for (int f = 0; f < D.F; ++f) sumn += D.widths[f];
  const size_t ea = esize(D.act), eb = esize(D.bank);
  const size_t nbank = (size_t)D.S * (size_t)D.rows * (size_t)D.ld;
  if (rows > 0) {
    const void* ptrs[] = {write_keys, read_queries, values, forget_gate, input_gate, subkeys, bank, snapshot,
                          grad_out, grad_bank, grad_write_keys, grad_read_queries, grad_values, grad_forget_gate,
                          grad_input_gate, grad_subkeys};
    const char* names[] = {"write_keys", "read_queries", "values", "forget_gate", "input_gate", "subkeys", "bank",
                           "snapshot", "grad_out", "grad_bank", "grad_write_keys", "grad_read_queries",
                           "grad_values", "grad_forget_gate", "grad_input_gate", "grad_subkeys"};
    for (int i = 0; i < 16; ++i) TRY(need(ptrs[i], names[i]));
  }
  TRY(aligned(bank, 16, "bank"));
  TRY(aligned(snapshot, 16, "snapshot"));
  TRY(aligned(grad_bank, 16, "grad_bank"));
  TRY(aligned(grad_values, 16, "grad_values"));
  const WsLayout L = layout(D, SDM_OP_BACKWARD);
  TRY(check_ws(workspace, workspace_bytes, L.total));
  const size_t qb = (size_t)rows * D.F * D.dk;
  const Range ins[] = {{write_keys, qb * ea, "write_keys"},
                       {read_queries, qb * ea, "read_queries"},
                       {values, (size_t)rows * D.d * ea, "values"},
                       {forget_gate, (size_t)rows * ea, "forget_gate"},
                       {input_gate, (size_t)rows * ea, "input_gate"},
                       {subkeys, (size_t)D.H * sumn * D.dk * ea, "subkeys"},
                       {snapshot, snapshot_bytes(D, snap_mode), "snapshot"},
                       {grad_out, (size_t)rows * D.d * ea, "grad_out"}};
  const Range outs[] = {{bank, nbank * eb, "bank"},
                        {grad_bank, nbank * (gb16 ? 2 : 4), "grad_bank"},
                        {grad_write_keys, qb * 4, "grad_write_keys"},
                        {grad_read_queries, qb * 4, "grad_read_queries"},
                        {grad_values, (size_t)rows * D.d * 4, "grad_values"},
                        {grad_forget_gate, (size_t)rows * 4, "grad_forget_gate"},
                        {grad_input_gate, (size_t)rows * 4, "grad_input_gate"},
                        {grad_subkeys, (size_t)D.H * sumn * D.dk * 4, "grad_subkeys"},
                        {workspace, L.total, "workspace"}};
  TRY(check_alias(outs, 9, ins, 8));
  TRY(check_device());
  if (rows == 0) return ok();
  hipStream_t st = (hipStream_t)stream;
  unsigned char* ws = (unsigned char*)workspace;
  const TopkPlan plans[2] = {pw, pr};
  TRY(hip_status(timed(SDM_K_CAND, st, [&] { return launch_cand_tables(plans, 2, D.F, (uint64_t*)(ws + L.cand), st); }),
                 "candidate table launch"));
  TopkArgs ta;
  memset(&ta, 0, sizeof ta);
  ta.queries[0] = write_keys;
  ta.queries[1] = read_queries;
  ta.subkeys = subkeys;
  ta.cand[0] = (const uint64_t*)(ws + L.cand);
  ta.cand[1] = (const uint64_t*)(ws + L.cand) + MAX_CAND;
  ta.plan[0] = pw;
  ta.plan[1] = pr;
  ta.nkinds = 2;
  ta.stream_major = 1;
  ta.ids[0] = (int32_t*)(ws + L.widx);
  ta.ids[1] = (int32_t*)(ws + L.ridx);
  ta.vals[0] = (float*)(ws + L.wwt);
  ta.vals[1] = (float*)(ws + L.rwt);
  ta.snorm = (float*)(ws + L.snorm);
  TRY(hip_status(timed(SDM_K_TOPK, st, [&] { return launch_topk(D, ta, st); }), "top-k launch"));
  BwdArgs ba;
  ba.widx = (const int32_t*)(ws + L.widx);
  ba.wwt = (const float*)(ws + L.wwt);
  ba.ridx = (const int32_t*)(ws + L.ridx);
  ba.rwt = (const float*)(ws + L.rwt);
  ba.wkeys = write_keys;
  ba.rq = read_queries;
  ba.subkeys = subkeys;
  ba.alpha = forget_gate;
  ba.beta = input_gate;
  ba.values = values;
  ba.gout = grad_out;
  ba.bank = bank;
  ba.snap = snapshot;
  ba.snap_mode = snap_mode;
  ba.gbank = grad_bank;
  ba.grad_bf16 = gb16 ? 1 : 0;
  ba.gwkeys = grad_write_keys;
  ba.grq = grad_read_queries;
  ba.gvalues = grad_values;
  ba.galpha = grad_forget_gate;
  ba.gbeta = grad_input_gate;
  ba.gsub = grad_subkeys;
  ba.part = (float*)(ws + L.part);
  ba.ds = (float*)(ws + L.ds);
  ba.sgpart = (float*)(ws + L.sgpart);
  ba.mrho = (float*)(ws + L.mrho);
  ba.mread = (float*)(ws + L.mread);
  const bool grouped = bwd_group_tokens(D) > 1;
  ba.gent = grouped ? (int32_t*)(ws + L.gent) : nullptr;
  ba.gcnt = grouped ? (int32_t*)(ws + L.gcnt) : nullptr;
  ba.giter = grouped ? (int32_t*)(ws + L.giter) : nullptr;
  ba.gn = grouped ? (int32_t*)(ws + L.gn) : nullptr;
  TRY(hip_status(timed(SDM_K_BWD, st, [&] { return launch_bwd(D, ba, st); }), "backward launch"));
  return ok();
}

sdm_status sdm_shared_bank_check(const sdm_config* cfg, const void* workspace, size_t workspace_bytes,
                                 int32_t* conflict, void* stream) {
  Dims D;
  TopkPlan pw, pr;
  TRY(validate(cfg, SDM_OP_WRITE_READ, 0, &D, &pw, &pr));
  if (!conflict) return fail(SDM_ERR_NULL, "conflict is NULL");
  if (!D.shared) return fail(SDM_ERR_RANGE, "cfg.shared_bank is 0: there is no shared-bank check to read");
  const WsLayout L = layout(D, SDM_OP_WRITE_READ);
  TRY(check_ws(workspace, workspace_bytes, L.total));
  TRY(check_device());
  *conflict = 0;
  if ((long long)D.B * D.T * D.H == 0) return ok();  // the op did no work
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return fail(SDM_ERR_HIP, "hipStreamSynchronize failed");
  int32_t flag = 0;
  if (hipMemcpy(&flag, (const unsigned char*)workspace + L.conflict, 4, hipMemcpyDeviceToHost) != hipSuccess)
    return fail(SDM_ERR_HIP, "reading the shared-bank flag failed");
  *conflict = flag != 0;
  return ok();
}

}  // extern "C"

// Scratch of sdm_decode_step_noalloc: one array per device, kept until the process ends. Host code never uses the
// array's name as an address (it is a host-side stand-in there); it uses the device address that
// hipGetSymbolAddress returned for the current device.
static __device__ __align__(256) unsigned char scratch[SDM_NOALLOC_SCRATCH_BYTES];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[64];

// The current device's address of `scratch`, looked up once per device (with that device current).
sdm_status scratch_address(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SDM_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(SDM_ERR_DEVICE, "device ordinal %d out of range [0, 64)", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(SDM_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return SDM_OK;
}

// The decode step with the caller's workspace, or (noalloc) with the device's scratch array in its place.
sdm_status decode_impl(const sdm_config* cfg, const void* write_keys, const void* read_queries, const void* values,
                       const void* forget_gate, const void* input_gate, const void* subkeys, const void* bank_in,
                       void* bank_out, void* out, int32_t* write_idx, int32_t* read_idx, void* workspace,
                       size_t workspace_bytes, void* stream, bool noalloc, bool steps = false) {
  Dims D;
  TopkPlan pw, pr;
  const int op = steps ? SDM_OP_DECODE_STEPS : SDM_OP_DECODE;
  TRY(validate(cfg, op, 0, &D, &pw, &pr));
  const long long rows = (long long)D.B * D.T * D.H;  // token rows (one token per stream for a single step)
  long long sumn = 0;
  for (int f = 0; f < D.F; ++f) sumn += D.widths[f];
  const size_t ea = esize(D.act), eb = esize(D.bank);
  const size_t bank_bytes = (size_t)D.S * (size_t)D.rows * (size_t)D.ld * eb;
  if (rows > 0) {
    TRY(need(write_keys, "write_keys"));
    TRY(need(read_queries, "read_queries"));
    TRY(need(values, "values"));
    TRY(need(forget_gate, "forget_gate"));
    TRY(need(input_gate, "input_gate"));
    TRY(need(subkeys, "subkeys"));
    TRY(need(bank_in, "bank_in"));
    TRY(need(bank_out, "bank_out"));
    TRY(need(out, "out"));
  }
  TRY(aligned(bank_in, 16, "bank_in"));
  TRY(aligned(bank_out, 16, "bank_out"));
  const WsLayout L = layout(D, op);
  if (noalloc) {
    if (L.total > SDM_NOALLOC_SCRATCH_BYTES)
      return fail(SDM_ERR_RANGE, "this decode step needs %zu bytes of scratch; sdm_decode_step_noalloc has %zu "
                  "(use sdm_decode_step with a workspace)", L.total, (size_t)SDM_NOALLOC_SCRATCH_BYTES);
  } else {
    TRY(check_ws(workspace, workspace_bytes, L.total));
  }
  const bool donated = bank_in == bank_out;
  const size_t qb = (size_t)rows * D.F * D.dk * ea;
  const Range ins[] = {{write_keys, qb, "write_keys"},
                       {read_queries, qb, "read_queries"},
                       {values, (size_t)rows * D.d * ea, "values"},
                       {forget_gate, (size_t)rows * ea, "forget_gate"},
                       {input_gate, (size_t)rows * ea, "input_gate"},
                       {subkeys, (size_t)D.H * sumn * D.dk * ea, "subkeys"},
                       {donated ? nullptr : bank_in, bank_bytes, "bank_in"}};
  const Range outs[] = {{bank_out, bank_bytes, "bank_out"},
                        {out, (size_t)rows * D.d * ea, "out"},
                        {write_idx, (size_t)rows * D.W * 4, "write_idx"},
                        {read_idx, (size_t)rows * D.R * 4, "read_idx"},
                        {noalloc ? nullptr : workspace, L.total, "workspace"}};
  TRY(check_alias(outs, 5, ins, 7));
  if (steps && rows > 0) {  // the steps kernel runs the one-launch step's arithmetic: only its shapes
    DecodeArgs probe;
    memset(&probe, 0, sizeof probe);
    probe.queries[0] = write_keys;
    probe.queries[1] = read_queries;
    probe.subkeys = subkeys;
    probe.plan[0] = pw;
    probe.plan[1] = pr;
    if (!decode_step_fits(D, probe))
      return fail(SDM_ERR_RANGE, "sdm_decode_steps runs the one-launch step's shapes only (num_writes, num_reads "
                  "<= 64, <= 256 sub-keys per factor, <= 1024 candidates, 16-byte aligned queries and sub-key rows): "
                  "use sdm_decode_step per token");
  }
  TRY(check_device());
  if (rows == 0) return ok();
  if (noalloc) TRY(scratch_address(&workspace));
  hipStream_t st = (hipStream_t)stream;
  unsigned char* ws = (unsigned char*)workspace;
  if (!donated)
    TRY(hip_status(timed(SDM_K_COPY, st, [&] { return launch_copy(bank_in, bank_out, bank_bytes, st); }),
                   "successor copy launch"));
  DecodeArgs a;
  memset(&a, 0, sizeof a);
  a.queries[0] = write_keys;
  a.queries[1] = read_queries;
  a.subkeys = subkeys;
  a.plan[0] = pw;
  a.plan[1] = pr;
  a.user_ids[0] = write_idx;
  a.user_ids[1] = read_idx;
  a.values = values;
  a.alpha = forget_gate;
  a.beta = input_gate;
  a.bank_in = bank_in;
  a.bank_out = bank_out;
  a.out = out;
  if (steps) {  // the batched top-k of every step, then the steps' rows in one launch
    const TopkPlan plans[2] = {pw, pr};
    TRY(hip_status(timed(SDM_K_CAND, st, [&] { return launch_cand_tables(plans, 2, D.F, (uint64_t*)(ws + L.cand), st); }),
                   "candidate table launch"));
    TopkArgs ta;
    memset(&ta, 0, sizeof ta);
    ta.queries[0] = write_keys;
    ta.queries[1] = read_queries;
    ta.subkeys = subkeys;
    ta.cand[0] = (const uint64_t*)(ws + L.cand);
    ta.cand[1] = (const uint64_t*)(ws + L.cand) + MAX_CAND;
    ta.plan[0] = pw;
    ta.plan[1] = pr;
    ta.nkinds = 2;
    ta.stream_major = 0;  // row-major [B, K, H, k] ids and float32 slot scores
    ta.ids[0] = (int32_t*)(ws + L.widx);
    ta.ids[1] = (int32_t*)(ws + L.ridx);
    ta.vals[0] = (float*)(ws + L.wwt);
    ta.vals[1] = (float*)(ws + L.rwt);
    ta.snorm = (float*)(ws + L.snorm);
    TRY(hip_status(timed(SDM_K_TOPK, st, [&] { return launch_topk(D, ta, st); }), "top-k launch"));
    a.wid = (const int32_t*)(ws + L.widx);
    a.wwt = (const float*)(ws + L.wwt);
    a.rid = (const int32_t*)(ws + L.ridx);
    a.rwt = (const float*)(ws + L.rwt);
    TRY(hip_status(timed(SDM_K_DECODE, st, [&] { return launch_decode_steps(D, a, D.T, st); }),
                   "decode steps launch"));
    return ok();
  }
  if (decode_step_fits(D, a)) {  // top-k, update and read in one launch
    TRY(hip_status(timed(SDM_K_DECODE, st, [&] { return launch_decode_step(D, a, st); }), "decode step launch"));
    return ok();
  }
  TopkArgs ta;
  memset(&ta, 0, sizeof ta);
  ta.queries[0] = write_keys;
  ta.queries[1] = read_queries;
  ta.subkeys = subkeys;
  ta.cand[0] = (const uint64_t*)(ws + L.cand);
  ta.cand[1] = (const uint64_t*)(ws + L.cand) + MAX_CAND;
  ta.plan[0] = pw;
  ta.plan[1] = pr;
  ta.nkinds = 2;
  ta.stream_major = 1;
  ta.ids[0] = (int32_t*)(ws + L.widx);
  ta.ids[1] = (int32_t*)(ws + L.ridx);
  ta.vals[0] = (float*)(ws + L.wwt);
  ta.vals[1] = (float*)(ws + L.rwt);
  ta.user_ids[0] = write_idx;
  ta.user_ids[1] = read_idx;
  ta.snorm = (float*)(ws + L.snorm);
  ta.one_query_per_wave = 1;
  TRY(hip_status(timed(SDM_K_TOPK, st, [&] { return launch_topk(D, ta, st); }), "top-k launch"));
  a.wid = (const int32_t*)(ws + L.widx);
  a.wwt = (const float*)(ws + L.wwt);
  a.rid = (const int32_t*)(ws + L.ridx);
  a.rwt = (const float*)(ws + L.rwt);
  TRY(hip_status(timed(SDM_K_DECODE, st, [&] { return launch_decode(D, a, st); }), "decode launch"));
  return ok();
}
}  // namespace

extern "C" {

sdm_status sdm_decode_step(const sdm_config* cfg, const void* write_keys, const void* read_queries,
                           const void* values, const void* forget_gate, const void* input_gate, const void* subkeys,
                           const void* bank_in, void* bank_out, void* out, int32_t* write_idx, int32_t* read_idx,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(cfg, write_keys, read_queries, values, forget_gate, input_gate, subkeys, bank_in, bank_out, out,
                     write_idx, read_idx, workspace, workspace_bytes, stream, false);
}

sdm_status sdm_decode_steps(const sdm_config* cfg, const void* write_keys, const void* read_queries,
                            const void* values, const void* forget_gate, const void* input_gate, const void* subkeys,
                            const void* bank_in, void* bank_out, void* out, int32_t* write_idx, int32_t* read_idx,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(cfg, write_keys, read_queries, values, forget_gate, input_gate, subkeys, bank_in, bank_out, out,
                     write_idx, read_idx, workspace, workspace_bytes, stream, false, true);
}

sdm_status sdm_decode_step_noalloc(const sdm_config* cfg, const void* write_keys, const void* read_queries,
                                   const void* values, const void* forget_gate, const void* input_gate,
                                   const void* subkeys, const void* bank_in, void* bank_out, void* out,
                                   int32_t* write_idx, int32_t* read_idx, void* stream) {
  return decode_impl(cfg, write_keys, read_queries, values, forget_gate, input_gate, subkeys, bank_in, bank_out, out,
                     write_idx, read_idx, nullptr, 0, stream, true);
}

// ------------------------------------------------------------------------------------------- layer (forward)
namespace {
struct LayerWs {
  size_t keys, queries, values, gin, alpha, beta, o, op, total;  // the forward (total: its workspace bytes)
  size_t opsize;                                                // the op region with the backward
  size_t dO, gk, gq, gv, gal, gbe, dp, tparam, w_outT, gyT, oT, xT, w_inT, dpT, btotal;  // the backward
  long long Mp, Np;                                             // B T and the input map's width, padded to 64
};
static sdm_status layer_layout(const sdm_layer_config* cfg, LayerWs* L) {
  if (!cfg) return fail(SDM_ERR_NULL, "cfg must not be NULL");
  if (cfg->reserved != 0) return fail(SDM_ERR_RANGE, "sdm_layer_config.reserved must be 0");
  if (cfg->op.shared_bank) return fail(SDM_ERR_RANGE, "the layer does not take a shared bank");
  size_t opws = 0;
  TRY(sdm_workspace_size(&cfg->op, SDM_OP_WRITE_READ, 0, &opws));
  if (cfg->op.act_dtype != SDM_BF16)
    return fail(SDM_ERR_DTYPE, "the layer computes in bfloat16 (act_dtype must be SDM_BF16)");
  const long long Dm = cfg->model_dim, H = cfg->op.heads, d = cfg->op.head_dim;
  if (Dm < 32 || Dm > 65536 || Dm % 32 != 0)
    return fail(SDM_ERR_RANGE, "model_dim = %lld must be a multiple of 32 in [32, 65536]", Dm);
  if ((H * d) % 32 != 0) return fail(SDM_ERR_RANGE, "heads * head_dim = %lld must be a multiple of 32", H * d);
  const long long M = (long long)cfg->op.batch * cfg->op.tokens;
  const long long P = (long long)cfg->op.num_factors * cfg->op.subkey_dim;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t r = o;
    o = (o + bytes + 255) & ~(size_t)255;
    return r;
  };
  L->keys = take((size_t)(M * H * P * 2));
  L->queries = take((size_t)(M * H * P * 2));
  L->values = take((size_t)(M * H * d * 2));
  L->gin = take((size_t)(M * 2 * H * 2));
  L->alpha = take((size_t)(M * H * 2));
  L->beta = take((size_t)(M * H * 2));
  L->o = take((size_t)(M * H * d * 2));
  L->op = take(opws);
  L->total = o;
  // the backward: the same prefix, the op region large enough for the op's backward, then its own regions (none
  // when the op has no backward for these settings: btotal 0, and the training calls refuse)
  size_t opb = 0;
  if (sdm_workspace_size(&cfg->op, SDM_OP_BACKWARD, 0, &opb) != SDM_OK) {
    L->opsize = opws;
    L->btotal = 0;
    return SDM_OK;
  }
  L->opsize = opb > opws ? opb : opws;
  o = L->op;
  take(L->opsize);
  const long long nin = 2 * H * P + H * d + 2 * H;
  L->Mp = (M + 63) / 64 * 64;
  L->Np = (nin + 63) / 64 * 64;
  L->dO = take((size_t)(M * H * d * 2));
  L->gk = take((size_t)(M * H * P * 4));
  L->gq = take((size_t)(M * H * P * 4));
  L->gv = take((size_t)(M * H * d * 4));
  L->gal = take((size_t)(M * H * 4));
  L->gbe = take((size_t)(M * H * 4));
  L->dp = take((size_t)(M * L->Np * 2));
  L->tparam = take((size_t)(2 * M * H * 4));
  L->w_outT = take((size_t)(H * d * Dm * 2));
  L->gyT = take((size_t)(Dm * L->Mp * 2));
  L->oT = take((size_t)(H * d * L->Mp * 2));
  L->xT = take((size_t)(Dm * L->Mp * 2));
  L->w_inT = take((size_t)(Dm * L->Np * 2));
  L->dpT = take((size_t)(L->Np * L->Mp * 2));
  L->btotal = o;
  return SDM_OK;
}
}  // namespace

sdm_status sdm_layer_workspace_size(const sdm_layer_config* cfg, size_t* bytes) {
  if (!bytes) return fail(SDM_ERR_NULL, "bytes must not be NULL");
  LayerWs L;
  TRY(layer_layout(cfg, &L));
  *bytes = L.total;
  return ok();
}

namespace {
static sdm_status layer_forward_impl(const sdm_layer_config* cfg, const void* x, const void* w_in, const float* a_log,
                              const float* dt_bias, const void* w_out, const void* subkeys, const void* initial_bank,
                              void* bank, void* y, void* snapshot, int32_t* write_idx, int32_t* read_idx,
                              void* workspace, size_t workspace_bytes, void* stream) {
  LayerWs L;
  TRY(layer_layout(cfg, &L));
  const sdm_config& oc = cfg->op;
  const long long M = (long long)oc.batch * oc.tokens, H = oc.heads, d = oc.head_dim, Dm = cfg->model_dim;
  const long long P = (long long)oc.num_factors * oc.subkey_dim;
  const long long nin = 2 * H * P + H * d + 2 * H;
  if (M > 0) {
    TRY(need(x, "x"));
    TRY(need(w_in, "w_in"));
    TRY(need(a_log, "a_log"));
    TRY(need(dt_bias, "dt_bias"));
    TRY(need(w_out, "w_out"));
    TRY(need(y, "y"));
  }
  if (M > 0) {
    TRY(need(subkeys, "subkeys"));
    TRY(need(bank, "bank"));
  }
  const void* al[] = {x, w_in, a_log, dt_bias, w_out, y, subkeys, bank, initial_bank};
  const char* an[] = {"x", "w_in", "a_log", "dt_bias", "w_out", "y", "subkeys", "bank", "initial_bank"};
  for (int i = 0; i < 9; ++i) TRY(aligned(al[i], 16, an[i]));
  TRY(check_ws(workspace, workspace_bytes, L.total));
  // the op's own checks (bank rows, pitch, ...) run here too, before any launch: a refused call does no work
  size_t opws = 0;
  TRY(sdm_workspace_size(&oc, SDM_OP_WRITE_READ, 0, &opws));
  long long sumn = 0;
  for (int f = 0; f < oc.num_factors; ++f) sumn += oc.factor_widths[f];
  const size_t eb = oc.bank_dtype == SDM_BF16 ? 2 : 4;
  const long long ld = oc.bank_row_stride ? oc.bank_row_stride : d;
  const size_t bank_bytes = (size_t)(oc.batch * H) * (size_t)oc.bank_rows * (size_t)ld * eb;
  const Range ins[] = {{x, (size_t)(M * Dm * 2), "x"},
                       {w_in, (size_t)(nin * Dm * 2), "w_in"},
                       {a_log, (size_t)H * 4, "a_log"},
                       {dt_bias, (size_t)H * 4, "dt_bias"},
                       {w_out, (size_t)(Dm * H * d * 2), "w_out"},
                       {subkeys, (size_t)(H * sumn * oc.subkey_dim * 2), "subkeys"},
                       {initial_bank, (size_t)H * (size_t)oc.bank_rows * (size_t)ld * eb, "initial_bank"}};
  size_t snap_bytes = 0;
  if (snapshot) TRY(sdm_snapshot_bytes(&oc, &snap_bytes));
  const Range outs[] = {{y, (size_t)(M * Dm * 2), "y"},
                        {workspace, L.total, "workspace"},
                        {bank, bank_bytes, "bank"},
                        {write_idx, (size_t)(M * H * oc.num_writes * 4), "write_idx"},
                        {read_idx, (size_t)(M * H * oc.num_reads * 4), "read_idx"},
                        {snapshot, snap_bytes, "snapshot"}};
  TRY(check_alias(outs, 6, ins, 7));
  TRY(check_device());
  if (M == 0 || H == 0) return ok();
  hipStream_t st = (hipStream_t)stream;
  unsigned char* ws = (unsigned char*)workspace;
  bf16_t* keys = (bf16_t*)(ws + L.keys);
  bf16_t* queries = (bf16_t*)(ws + L.queries);
  bf16_t* values = (bf16_t*)(ws + L.values);
  bf16_t* gin = (bf16_t*)(ws + L.gin);
  bf16_t* alpha = (bf16_t*)(ws + L.alpha);
  bf16_t* beta = (bf16_t*)(ws + L.beta);
  bf16_t* o = (bf16_t*)(ws + L.o);
  GemmArgs g;
  memset(&g, 0, sizeof g);
  g.x = (const bf16_t*)x;
  g.w = (const bf16_t*)w_in;
  g.M = (int)M;
  g.N = (int)nin;
  g.K = (int)Dm;
  g.nseg = 4;
  g.seg[0] = {(int)(H * P), keys, (int)(H * P)};
  g.seg[1] = {(int)(2 * H * P), queries, (int)(H * P)};
  g.seg[2] = {(int)(2 * H * P + H * d), values, (int)(H * d)};
  g.seg[3] = {(int)nin, gin, (int)(2 * H)};
  TRY(hip_status(timed(SDM_K_DENSE, st, [&] { return launch_gemm_bf16(g, st); }), "projection launch"));
  TRY(hip_status(timed(SDM_K_DENSE, st, [&] {
                   return launch_gates(gin, gin + H, (int)(2 * H), a_log, dt_bias, M * H, (int)H, alpha, beta, st);
                 }),
                 "gates launch"));
  if (initial_bank) {  // the per-sequence copy of the learned bank into every batch row
    long long N = 1;
    for (int f = 0; f < oc.num_factors; ++f) N *= oc.factor_widths[f];
    TRY(hip_status(launch_bank_broadcast(initial_bank, bank, oc.batch, (int)H, N, oc.bank_rows, (int)d, ld, (int)eb,
                                         st),
                   "bank copy launch"));
  }
  TRY(write_read_impl(&oc, keys, queries, values, alpha, beta, subkeys, bank, o, snapshot, write_idx, read_idx,
                      ws + L.op, workspace_bytes - L.op, stream));
  GemmArgs go;
  memset(&go, 0, sizeof go);
  go.x = o;
  go.w = (const bf16_t*)w_out;
  go.M = (int)M;
  go.N = (int)Dm;
  go.K = (int)(H * d);
  go.nseg = 1;
  go.seg[0] = {(int)Dm, (bf16_t*)y, (int)Dm};
  TRY(hip_status(timed(SDM_K_DENSE, st, [&] { return launch_gemm_bf16(go, st); }), "output projection launch"));
  return ok();
}
}  // namespace

sdm_status sdm_layer_forward(const sdm_layer_config* cfg, const void* x, const void* w_in, const float* a_log,
                             const float* dt_bias, const void* w_out, const void* subkeys, const void* initial_bank,
                             void* bank, void* y, int32_t* write_idx, int32_t* read_idx, void* workspace,
                             size_t workspace_bytes, void* stream) {
  return layer_forward_impl(cfg, x, w_in, a_log, dt_bias, w_out, subkeys, initial_bank, bank, y, nullptr, write_idx,
                            read_idx, workspace, workspace_bytes, stream);
}

sdm_status sdm_layer_forward_save(const sdm_layer_config* cfg, const void* x, const void* w_in, const float* a_log,
                                  const float* dt_bias, const void* w_out, const void* subkeys,
                                  const void* initial_bank, void* bank, void* y, void* snapshot, int32_t* write_idx,
                                  int32_t* read_idx, void* workspace, size_t workspace_bytes, void* stream) {
  if (cfg && (long long)cfg->op.batch * cfg->op.tokens * cfg->op.heads > 0 && !snapshot)
    return fail(SDM_ERR_NULL, "snapshot is NULL");
  size_t need_ws = 0;
  TRY(sdm_layer_backward_workspace_size(cfg, &need_ws));
  TRY(check_ws(workspace, workspace_bytes, need_ws));  // the backward's workspace: the backward reads this one
  return layer_forward_impl(cfg, x, w_in, a_log, dt_bias, w_out, subkeys, initial_bank, bank, y, snapshot,
                            write_idx, read_idx, workspace, workspace_bytes, stream);
}

sdm_status sdm_layer_backward_workspace_size(const sdm_layer_config* cfg, size_t* bytes) {
  if (!bytes) return fail(SDM_ERR_NULL, "bytes must not be NULL");
  LayerWs L;
  TRY(layer_layout(cfg, &L));
  if (L.btotal == 0) {  // the op's own refusal, with its message
    size_t opb = 0;
    return sdm_workspace_size(&cfg->op, SDM_OP_BACKWARD, 0, &opb);
  }
  size_t sb = 0;
  TRY(sdm_snapshot_bytes(&cfg->op, &sb));  // the snapshot's route (cfg.op.snapshot_dtype) refused here already
  *bytes = L.btotal;
  return ok();
}

sdm_status sdm_layer_backward(const sdm_layer_config* cfg, const void* x, const void* w_in, const float* a_log,
                              const float* dt_bias, const void* w_out, const void* subkeys, void* bank,
                              const void* snapshot, const void* grad_y, void* grad_bank, float* grad_x,
                              float* grad_w_in, float* grad_a_log, float* grad_dt_bias, float* grad_w_out,
                              float* grad_subkeys, void* workspace, size_t workspace_bytes, void* stream) {
  LayerWs L;
  TRY(layer_layout(cfg, &L));
  size_t need_ws = 0;
  TRY(sdm_layer_backward_workspace_size(cfg, &need_ws));
  const sdm_config& oc = cfg->op;
  const long long M = (long long)oc.batch * oc.tokens, H = oc.heads, d = oc.head_dim, Dm = cfg->model_dim;
  const long long P = (long long)oc.num_factors * oc.subkey_dim, Hd = H * d;
  const long long nin = 2 * H * P + Hd + 2 * H;
  if (M > 0) {
    const void* ptrs[] = {x, w_in, a_log, dt_bias, w_out, subkeys, bank, snapshot, grad_y, grad_bank, grad_x,
                          grad_w_in, grad_a_log, grad_dt_bias, grad_w_out, grad_subkeys};
    const char* names[] = {"x", "w_in", "a_log", "dt_bias", "w_out", "subkeys", "bank", "snapshot", "grad_y",
                           "grad_bank", "grad_x", "grad_w_in", "grad_a_log", "grad_dt_bias", "grad_w_out",
                           "grad_subkeys"};
    for (int i = 0; i < 16; ++i) TRY(need(ptrs[i], names[i]));
  }
  const void* al[] = {x, w_in, w_out, grad_y, grad_x, grad_w_in, grad_w_out};
  const char* an[] = {"x", "w_in", "w_out", "grad_y", "grad_x", "grad_w_in", "grad_w_out"};
  for (int i = 0; i < 7; ++i) TRY(aligned(al[i], 16, an[i]));
  TRY(check_ws(workspace, workspace_bytes, L.btotal));
  // the op's own checks (dtypes, snapshot route, gradient dtype, ...) before any launch
  Dims D;
  TopkPlan pw, pr;
  TRY(validate(&oc, SDM_OP_BACKWARD, 0, &D, &pw, &pr));
  int snap_mode = SNAP_BANK;
  TRY(snapshot_kind(&oc, D, &snap_mode));
  bool gb16 = false;
  TRY(grad_bank_kind(&oc, D, true, &gb16));
  long long sumn = 0;
  for (int f = 0; f < oc.num_factors; ++f) sumn += oc.factor_widths[f];
  const size_t nbank = (size_t)D.S * (size_t)D.rows * (size_t)D.ld;
  const Range ins[] = {{x, (size_t)(M * Dm * 2), "x"},
                       {w_in, (size_t)(nin * Dm * 2), "w_in"},
                       {a_log, (size_t)H * 4, "a_log"},
                       {dt_bias, (size_t)H * 4, "dt_bias"},
                       {w_out, (size_t)(Dm * Hd * 2), "w_out"},
                       {subkeys, (size_t)(H * sumn * oc.subkey_dim * 2), "subkeys"},
                       {snapshot, snapshot_bytes(D, snap_mode), "snapshot"},
                       {grad_y, (size_t)(M * Dm * 2), "grad_y"}};
  const Range outs[] = {{bank, nbank * esize(D.bank), "bank"},
                        {grad_bank, nbank * (gb16 ? 2 : 4), "grad_bank"},
                        {grad_x, (size_t)(M * Dm * 4), "grad_x"},
                        {grad_w_in, (size_t)(nin * Dm * 4), "grad_w_in"},
                        {grad_a_log, (size_t)H * 4, "grad_a_log"},
                        {grad_dt_bias, (size_t)H * 4, "grad_dt_bias"},
                        {grad_w_out, (size_t)(Dm * Hd * 4), "grad_w_out"},
                        {grad_subkeys, (size_t)(H * sumn * oc.subkey_dim * 4), "grad_subkeys"},
                        {workspace, L.btotal, "workspace"}};
  TRY(check_alias(outs, 9, ins, 8));
  TRY(check_device());
  if (M == 0 || H == 0) return ok();
  hipStream_t st = (hipStream_t)stream;
  unsigned char* ws = (unsigned char*)workspace;
  const bf16_t* gy = (const bf16_t*)grad_y;
  auto transpose = [&](const void* in, long long R, long long C, long long ldi, size_t off, long long Rp) {
    return hip_status(timed(SDM_K_DENSE, st, [&] {
                        return launch_transpose_bf16((const bf16_t*)in, (int)R, (int)C, ldi, (bf16_t*)(ws + off),
                                                     (int)Rp, Rp, st);
                      }),
                      "transpose launch");
  };
  auto gemm = [&](const void* xa, size_t wt, long long m, long long n, long long k, void* dst, bool f32) {
    GemmArgs g;
    memset(&g, 0, sizeof g);
    g.x = (const bf16_t*)xa;
    g.w = (const bf16_t*)(ws + wt);
    g.M = (int)m;
    g.N = (int)n;
    g.K = (int)k;
    g.nseg = 1;
    if (f32) {
      g.f32 = (float*)dst;
      g.f32ld = n;
    } else {
      g.seg[0] = {(int)n, (bf16_t*)dst, (int)n};
    }
    return hip_status(timed(SDM_K_DENSE, st, [&] { return launch_gemm_bf16(g, st); }), "dense map launch");
  };
  // the output map: d o = grad_y w_out (bfloat16), d w_out = grad_y^T o
  TRY(transpose(w_out, Dm, Hd, Hd, L.w_outT, Dm));
  TRY(transpose(grad_y, M, Dm, Dm, L.gyT, L.Mp));
  TRY(transpose(ws + L.o, M, Hd, Hd, L.oT, L.Mp));
  TRY(gemm(gy, L.w_outT, M, Hd, Dm, ws + L.dO, false));
  TRY(gemm(ws + L.gyT, L.oT, Dm, Hd, L.Mp, grad_w_out, true));
  // the op's backward on d o, from the activations the forward left in the workspace
  TRY(sdm_write_read_backward(&oc, ws + L.keys, ws + L.queries, ws + L.values, ws + L.alpha, ws + L.beta, subkeys,
                              bank, snapshot, ws + L.dO, grad_bank, (float*)(ws + L.gk), (float*)(ws + L.gq),
                              (float*)(ws + L.gv), (float*)(ws + L.gal), (float*)(ws + L.gbe), grad_subkeys,
                              ws + L.op, L.opsize, stream));
  // the gates' derivatives and d p (bfloat16), then the input map: d x = d p w_in, d w_in = d p^T x
  GateBwdArgs ga;
  ga.gk = (const float*)(ws + L.gk);
  ga.gq = (const float*)(ws + L.gq);
  ga.gv = (const float*)(ws + L.gv);
  ga.galpha = (const float*)(ws + L.gal);
  ga.gbeta = (const float*)(ws + L.gbe);
  ga.gin = (const bf16_t*)(ws + L.gin);
  ga.a_log = a_log;
  ga.dt_bias = dt_bias;
  ga.dp = (bf16_t*)(ws + L.dp);
  ga.tparam = (float*)(ws + L.tparam);
  ga.M = M;
  ga.H = (int)H;
  ga.HP = (int)(H * P);
  ga.Hd = (int)Hd;
  ga.ldp = (int)L.Np;
  TRY(hip_status(timed(SDM_K_DENSE, st, [&] { return launch_layer_grad_assemble(ga, st); }), "gate gradient launch"));
  TRY(hip_status(timed(SDM_K_DENSE, st, [&] {
                   return launch_layer_param_sums((const float*)(ws + L.tparam), M, (int)H, grad_a_log, grad_dt_bias,
                                                  st);
                 }),
                 "gate parameter sum launch"));
  TRY(transpose(w_in, nin, Dm, Dm, L.w_inT, L.Np));
  TRY(transpose(ws + L.dp, M, L.Np, L.Np, L.dpT, L.Mp));
  TRY(transpose(x, M, Dm, Dm, L.xT, L.Mp));
  TRY(gemm(ws + L.dp, L.w_inT, M, Dm, L.Np, grad_x, true));
  TRY(gemm(ws + L.dpT, L.xT, nin, Dm, L.Mp, grad_w_in, true));
  return ok();
}

sdm_status sdm_snapshot_bytes(const sdm_config* cfg, size_t* bytes) {
  if (!bytes) return fail(SDM_ERR_NULL, "bytes must not be NULL");
  Dims D;
  TopkPlan pw, pr;
  TRY(validate(cfg, SDM_OP_BACKWARD, 0, &D, &pw, &pr));
  int mode = SNAP_BANK;
  TRY(snapshot_kind(cfg, D, &mode));
  *bytes = snapshot_bytes(D, mode);
  return ok();
}

sdm_status sdm_bank_grad_sum(const sdm_config* cfg, const void* grad_bank, float* grad_initial_bank,
                             void* stream) {
  Dims D;
  TopkPlan pw, pr;
  TRY(validate(cfg, SDM_OP_WRITE_READ, 0, &D, &pw, &pr));
  bool gb16 = false;
  TRY(grad_bank_kind(cfg, D, false, &gb16));
  if (D.shared) return fail(SDM_ERR_RANGE, "sdm_bank_grad_sum takes per-stream bank gradients (shared_bank = 0)");
  if (D.S > 0) {
    TRY(need(grad_bank, "grad_bank"));
    TRY(need(grad_initial_bank, "grad_initial_bank"));
  }
  TRY(aligned(grad_bank, 16, "grad_bank"));
  TRY(aligned(grad_initial_bank, 16, "grad_initial_bank"));
  if ((D.ld * 4) % 16 != 0 || D.d % 4 != 0)
    return fail(SDM_ERR_LAYOUT, "the bank gradient's rows must be 16-byte multiples (head_dim and row stride)");
  const size_t row_bytes = (size_t)D.rows * (size_t)D.ld * 4;
  const Range ins[] = {{grad_bank, (size_t)D.S * row_bytes / (gb16 ? 2 : 1), "grad_bank"}};
  const Range outs[] = {{grad_initial_bank, (size_t)D.H * row_bytes, "grad_initial_bank"}};
  TRY(check_alias(outs, 1, ins, 1));
  TRY(check_device());
  if (D.S == 0) return ok();
  TRY(hip_status(launch_bank_grad_sum(grad_bank, gb16, grad_initial_bank, D.B, D.H, D.N, D.rows, D.d, D.ld,
                                      (hipStream_t)stream),
                 "bank gradient sum launch"));
  return ok();
}

sdm_status sdm_profile_enable(int32_t on) {
  std::lock_guard<std::mutex> g(g_prof_mu);
  for (auto& p : g_prof_pending) {
    g_prof_pool.push_back(p.a);
    g_prof_pool.push_back(p.b);
  }
  g_prof_pending.clear();
  for (int k = 0; k < SDM_K_COUNT; ++k) {
    g_prof_ms[k] = 0.0;
    g_prof_n[k] = 0;
  }
  g_prof_on = on != 0;
  return ok();
}

sdm_status sdm_profile_read(double* ms, int64_t* launches) {
  if (!ms || !launches) return fail(SDM_ERR_NULL, "ms and launches must not be NULL");
  std::lock_guard<std::mutex> g(g_prof_mu);
  for (auto& p : g_prof_pending) {
    float t = 0.0f;
    if (hipEventSynchronize(p.b) != hipSuccess || hipEventElapsedTime(&t, p.a, p.b) != hipSuccess)
      return fail(SDM_ERR_HIP, "reading kernel timing events failed");
    g_prof_ms[p.kernel] += t;
    g_prof_n[p.kernel] += 1;
    g_prof_pool.push_back(p.a);
    g_prof_pool.push_back(p.b);
  }
  g_prof_pending.clear();
  for (int k = 0; k < SDM_K_COUNT; ++k) {
    ms[k] = g_prof_ms[k];
    launches[k] = g_prof_n[k];
  }
  return ok();
}

}  // extern "C"
