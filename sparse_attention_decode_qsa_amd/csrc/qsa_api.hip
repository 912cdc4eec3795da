// qsa_api.hip - the C ABI of libqsa: argument checks, workspace sizing, launches.
// Every check that can be made on the host runs before anything is enqueued.
#include <mutex>

#include "../../include/qsa.h"
#include "qsa_device.h"

// Static scratch of qsa_decode_noalloc (the workspace of the decode chain for callers that
// cannot allocate). On the host the name is only a stand-in for the symbol: kernels get the
// device address that hipGetSymbolAddress returns for the current device, never the name.
static __device__ __align__(256) unsigned char scratch[QSA_NOALLOC_SCRATCH_BYTES];

namespace qsa {
hipError_t launch_index_score(const int8_t*, const int8_t*, const int32_t*, const int32_t*, int, int,
                              int, int32_t*, int32_t*, int, hipStream_t);   // ..., T, stream
hipError_t launch_multi_scan(const int8_t*, const int8_t*, const int32_t*, const int32_t*, int, int, int,
                             int32_t*, int32_t*, int, hipStream_t);         // ..., T, stream
void set_scan_events(hipEvent_t start, hipEvent_t stop);
size_t topk_workspace_bytes(int B, int max_blocks);
constexpr int kMaxSelBlocks = 262144;
hipError_t launch_topk_select(const int32_t*, const int32_t*, const int32_t*, int, int, int, int, int32_t*,
                              int32_t*, int, hipStream_t);                  // ..., T, stream
size_t attn_workspace_bytes(int B, int Hq, int Hkv, int P);
hipError_t launch_sparse_attn(const void*, const void*, const void*, const int32_t*, const int32_t*,
                              const int32_t*, const int32_t*, int, int, int, int, int, int, float, float*,
                              float*, float*, float*, void*, int, hipStream_t);  // ..., workspace, T, stream
hipError_t launch_lse_merge(const float*, const float*, int, int, int, float*, float*, hipStream_t);
hipError_t launch_check_pages(const int32_t*, const int32_t*, int, int, int, int, int32_t*, hipStream_t);
hipError_t launch_pool_build(const int8_t*, const int32_t*, const int32_t*, int, int, int16_t*, hipStream_t);
hipError_t launch_cache_append(const void*, const void*, const int8_t*, const int32_t*, void*, void*, int8_t*,
                               int16_t*, const int32_t*, const int32_t*, int, int, int, hipStream_t);
hipError_t launch_index_score_pooled(const int8_t*, const int16_t*, const int32_t*, const int32_t*, int, int, int,
                                     int32_t*, int32_t*, const void*, const void*, const int8_t*, const int32_t*,
                                     void*, void*, int8_t*, int, hipStream_t, int T, const int8_t* idx_keys);

namespace {

thread_local int g_last_hip_error = 0;

qsa_status_t hip_status(hipError_t e) {
  if (e == hipSuccess) return QSA_OK;
  g_last_hip_error = (int)e;
  return QSA_ERR_HIP;
}

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

qsa_status_t check_index(const int8_t* q_idx, const int8_t* idx_cache, const int32_t* page_table,
                         const int32_t* lens, int B, int n_idx_heads, int idx_dim, int page_size,
                         int max_pages, int max_blocks, const int32_t* scores) {
  if (B < 0 || max_pages < 1 || max_blocks < 1) return QSA_ERR_SHAPE;
  if (n_idx_heads != kIdxHeads || idx_dim != kIdxDim || page_size != kPageSize) return QSA_ERR_UNSUPPORTED;
  if ((long long)max_blocks < (long long)max_pages * kBlocksPerPage) return QSA_ERR_SHAPE;
  if (B > 65535) return QSA_ERR_UNSUPPORTED;
  if (B == 0) return QSA_OK;
  if (!q_idx || !idx_cache || !page_table || !lens || !scores) return QSA_ERR_NULL;
  if (misaligned(q_idx) || misaligned(idx_cache)) return QSA_ERR_SHAPE;
  return QSA_OK;
}

qsa_status_t check_topk(const int32_t* scores, const int32_t* lens, int B, int max_blocks, int k,
                        const int32_t* sel, const int32_t* cnt) {
  if (B < 0 || max_blocks < 1 || k < 1) return QSA_ERR_SHAPE;
  if (k > kMaxK || max_blocks > kMaxSelBlocks) return QSA_ERR_UNSUPPORTED;
  if (B > 65535) return QSA_ERR_UNSUPPORTED;
  if (max_blocks % 4 != 0) return QSA_ERR_SHAPE;
  if (B == 0) return QSA_OK;
  if (!scores || !lens || !sel || !cnt) return QSA_ERR_NULL;
  if (misaligned(scores)) return QSA_ERR_SHAPE;
  return QSA_OK;
}

qsa_status_t check_attn(const void* q, const void* kc, const void* vc, const int32_t* page_table,
                        const int32_t* lens, const int32_t* sel, const int32_t* cnt, int B, int Hq,
                        int Hkv, int head_dim, int page_size, int max_pages, int k, int P,
                        const float* po, const float* pl) {
  if (B < 0 || Hq < 1 || Hkv < 1 || max_pages < 1 || k < 1 || P < 1) return QSA_ERR_SHAPE;
  if (Hq % Hkv != 0) return QSA_ERR_SHAPE;
  if (head_dim != kHeadDim || page_size != kPageSize) return QSA_ERR_UNSUPPORTED;
  if (Hq / Hkv > kMaxGroup || k > kMaxK || P > kMaxSlices) return QSA_ERR_UNSUPPORTED;
  if (B > 65535 || Hkv > 65535) return QSA_ERR_UNSUPPORTED;
  if (B == 0) return QSA_OK;
  if (!q || !kc || !vc || !page_table || !lens || !sel || !cnt || !po || !pl) return QSA_ERR_NULL;
  if (misaligned(q) || misaligned(kc) || misaligned(vc) || misaligned(po)) return QSA_ERR_SHAPE;
  return QSA_OK;
}

qsa_status_t check_merge(const float* po, const float* pl, int B, int P, int Hq, int head_dim,
                         const float* out) {
  if (B < 0 || P < 1 || Hq < 1) return QSA_ERR_SHAPE;
  if (head_dim != kHeadDim) return QSA_ERR_UNSUPPORTED;
  if (B > 65535 || Hq > 65535) return QSA_ERR_UNSUPPORTED;
  if (B == 0) return QSA_OK;
  if (!po || !pl || !out) return QSA_ERR_NULL;
  if (misaligned(out)) return QSA_ERR_SHAPE;
  return QSA_OK;
}

// A workspace of `need` bytes: may be NULL when nothing is needed.
bool workspace_ok(const void* ws, size_t have, size_t need) {
  return need == 0 || (ws != nullptr && have >= need);
}

__global__ void zero_fill_kernel(uint32_t* p, size_t nwords) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < nwords; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

}  // namespace
}  // namespace qsa

using namespace qsa;

extern "C" {

const char* qsa_status_string(int s) {
  switch (s) {
    case QSA_OK: return "ok";
    case QSA_ERR_NULL: return "a required pointer is NULL";
    case QSA_ERR_SHAPE: return "sizes are negative or inconsistent";
    case QSA_ERR_UNSUPPORTED: return "size outside the compiled kernel shapes";
    case QSA_ERR_WORKSPACE: return "workspace missing or too small";
    case QSA_ERR_HIP: return "HIP runtime error";
    case QSA_ERR_SCRATCH: return "the call needs more workspace than the static scratch holds";
    default: return "unknown status";
  }
}

int qsa_last_hip_error(void) { return g_last_hip_error; }

qsa_status_t qsa_time_next_scan(void* start_event, void* stop_event) {
  set_scan_events(static_cast<hipEvent_t>(start_event), static_cast<hipEvent_t>(stop_event));
  return QSA_OK;
}

int qsa_version(void) { return 230; }   // 0.2.3: nontemporal score stores in chunks of 5-64 new tokens

qsa_status_t qsa_index_score(const int8_t* q_idx, const int8_t* idx_cache, const int32_t* page_table,
                             const int32_t* context_lens, int B, int n_idx_heads, int idx_dim,
                             int page_size, int max_pages_per_seq, int max_blocks,
                             int32_t* block_scores, int32_t* page_max, void* stream) {
  qsa_status_t st = check_index(q_idx, idx_cache, page_table, context_lens, B, n_idx_heads, idx_dim,
                                page_size, max_pages_per_seq, max_blocks, block_scores);
  if (st != QSA_OK || B == 0) return st;
  return hip_status(launch_index_score(q_idx, idx_cache, page_table, context_lens, B, max_pages_per_seq,
                                       max_blocks, block_scores, page_max, 1, (hipStream_t)stream));
}

size_t qsa_topk_workspace_size(int B, int max_blocks, int k) {
  (void)k;
  if (B <= 0 || max_blocks <= 0) return 0;
  return topk_workspace_bytes(B, max_blocks);
}

qsa_status_t qsa_topk_select(const int32_t* block_scores, const int32_t* context_lens,
                             const int32_t* page_max, int B, int max_blocks, int max_pages_per_seq, int k,
                             int32_t* sel_blocks, int32_t* sel_count, void* workspace,
                             size_t workspace_bytes, void* stream) {
  qsa_status_t st = check_topk(block_scores, context_lens, B, max_blocks, k, sel_blocks, sel_count);
  if (st == QSA_OK && page_max && (max_pages_per_seq < 1 ||
                                   (long long)max_pages_per_seq * kBlocksPerPage < (long long)max_blocks - 15))
    st = QSA_ERR_SHAPE;
  if (st != QSA_OK || B == 0) return st;
  if (!workspace_ok(workspace, workspace_bytes, topk_workspace_bytes(B, max_blocks))) return QSA_ERR_WORKSPACE;
  return hip_status(launch_topk_select(block_scores, context_lens, page_max, B, max_blocks,
                                       max_pages_per_seq, k, sel_blocks, sel_count, 1, (hipStream_t)stream));
}

size_t qsa_attn_workspace_size(int B, int Hq, int Hkv, int k, int P) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || k <= 0 || P <= 0) return 0;
  return attn_workspace_bytes(B, Hq, Hkv, P);
}

qsa_status_t qsa_sparse_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* page_table, const int32_t* context_lens,
                                    const int32_t* sel_blocks, const int32_t* sel_count, int B, int Hq,
                                    int Hkv, int head_dim, int page_size, int max_pages_per_seq, int k,
                                    int P, float softmax_scale, float* partial_out, float* partial_lse,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  qsa_status_t st = check_attn(q, k_cache, v_cache, page_table, context_lens, sel_blocks, sel_count, B,
                               Hq, Hkv, head_dim, page_size, max_pages_per_seq, k, P, partial_out,
                               partial_lse);
  if (st != QSA_OK || B == 0) return st;
  if (!workspace_ok(workspace, workspace_bytes, attn_workspace_bytes(B, Hq, Hkv, P))) return QSA_ERR_WORKSPACE;
  if (misaligned(workspace)) return QSA_ERR_SHAPE;
  return hip_status(launch_sparse_attn(q, k_cache, v_cache, page_table, context_lens, sel_blocks,
                                       sel_count, B, Hq, Hkv, max_pages_per_seq, k, P, softmax_scale,
                                       partial_out, partial_lse, nullptr, nullptr, workspace, 1,
                                       (hipStream_t)stream));
}

qsa_status_t qsa_lse_merge(const float* partial_out, const float* partial_lse, int B, int P, int Hq,
                           int head_dim, float* out, float* out_lse, void* stream) {
  qsa_status_t st = check_merge(partial_out, partial_lse, B, P, Hq, head_dim, out);
  if (st != QSA_OK || B == 0) return st;
  return hip_status(launch_lse_merge(partial_out, partial_lse, B, P, Hq, out, out_lse, (hipStream_t)stream));
}

// qsa_decode's workspace: the per-page maxima [B, max_blocks/16] int32 (written by the
// indexer scan, read by the selection), then the attention workspace (partials of the
// shares of every slice, written by the attention kernel, read by the merge).
size_t decode_pm_bytes(int B, int max_blocks) {
  return align256((size_t)B * ((max_blocks + kBlocksPerPage - 1) / kBlocksPerPage) * sizeof(int32_t));
}

size_t qsa_decode_workspace_size(int B, int Hq, int Hkv, int max_blocks, int k, int P) {
  if (B <= 0 || max_blocks <= 0) return 0;
  return decode_pm_bytes(B, max_blocks) + align256(qsa_topk_workspace_size(B, max_blocks, k)) +
         qsa_attn_workspace_size(B, Hq, Hkv, k, P);
}

namespace {

// The decode step's cache writes, made by the pooled scan (qsa_decode_step_pooled).
struct StepIn {
  const void* k_new;
  const void* v_new;
  const int8_t* idx_new;
  const int32_t* write;
  void* k_cache;
  void* v_cache;
  int8_t* idx_cache;
};

// The chain of qsa_decode, qsa_decode_pooled, qsa_decode_step_pooled, qsa_decode_multi and
// qsa_decode_multi_pooled: the scan reads idx_cache (int8 keys, T draft queries per request)
// or, when pooled is given, the side cache of pooled keys (and makes the step's cache writes
// when step is given; with 2 <= T <= 4 draft tokens it also reads idx_cache on the pages that
// hold draft positions); the selection, attention and merge run on the B*T virtual requests.
qsa_status_t decode_chain(const void* q, const int8_t* q_idx, const int8_t* idx_cache, const int16_t* pooled,
                          const void* k_cache, const void* v_cache, const int32_t* page_table,
                          const int32_t* context_lens, int B, int T, int Hq, int Hkv, int head_dim, int n_idx_heads,
                          int idx_dim, int page_size, int max_pages_per_seq, int max_blocks, int k, int P,
                          float softmax_scale, int32_t* block_scores, int32_t* sel_blocks, int32_t* sel_count,
                          float* partial_out, float* partial_lse, float* out, float* out_lse, void* workspace,
                          size_t workspace_bytes, void* stream, const StepIn* step = nullptr) {
  const int8_t* keys = pooled ? reinterpret_cast<const int8_t*>(pooled) : idx_cache;
  if (T < 1 || (pooled && step && T != 1)) return QSA_ERR_SHAPE;
  if (T > kMaxQueries || (pooled && T > 4)) return QSA_ERR_UNSUPPORTED;
  if (pooled && T > 1 && B > 0 && (!idx_cache || misaligned(idx_cache))) return idx_cache ? QSA_ERR_SHAPE : QSA_ERR_NULL;
  const int BT = B * T;   // virtual requests (request, draft token)
  qsa_status_t st = check_index(q_idx, keys, page_table, context_lens, B, n_idx_heads, idx_dim, page_size,
                                max_pages_per_seq, max_blocks, block_scores);
  if (st == QSA_OK) st = check_topk(block_scores, context_lens, BT, max_blocks, k, sel_blocks, sel_count);
  if (st == QSA_OK)
    st = check_attn(q, k_cache, v_cache, page_table, context_lens, sel_blocks, sel_count, BT, Hq, Hkv,
                    head_dim, page_size, max_pages_per_seq, k, P, partial_out, partial_lse);
  if (st == QSA_OK) st = check_merge(partial_out, partial_lse, BT, P, Hq, head_dim, out);
  if (st != QSA_OK || B == 0) return st;
  const size_t pmb = decode_pm_bytes(BT, max_blocks);
  const size_t tb = align256(topk_workspace_bytes(BT, max_blocks));
  if (!workspace_ok(workspace, workspace_bytes, pmb + tb + attn_workspace_bytes(BT, Hq, Hkv, P)))
    return QSA_ERR_WORKSPACE;
  if (misaligned(workspace)) return QSA_ERR_SHAPE;
  int32_t* page_max = static_cast<int32_t*>(workspace);   // [BT, max_pages_per_seq] fits: 16*max_pages <= max_blocks
  char* ws_attn = static_cast<char*>(workspace) + pmb + tb;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = pooled ? launch_index_score_pooled(q_idx, pooled, page_table, context_lens, B, max_pages_per_seq,
                                                    max_blocks, block_scores, page_max,
                                                    step ? step->k_new : nullptr, step ? step->v_new : nullptr,
                                                    step ? step->idx_new : nullptr, step ? step->write : nullptr,
                                                    step ? step->k_cache : nullptr, step ? step->v_cache : nullptr,
                                                    step ? step->idx_cache : nullptr, Hkv, s, T, idx_cache)
                        : launch_multi_scan(q_idx, idx_cache, page_table, context_lens, B, max_pages_per_seq,
                                            max_blocks, block_scores, page_max, T, s);
  if (e == hipSuccess)
    e = launch_topk_select(block_scores, context_lens, page_max, BT, max_blocks, max_pages_per_seq, k,
                           sel_blocks, sel_count, T, s);
  if (e == hipSuccess)
    e = launch_sparse_attn(q, k_cache, v_cache, page_table, context_lens, sel_blocks, sel_count, BT, Hq, Hkv,
                           max_pages_per_seq, k, P, softmax_scale, partial_out, partial_lse, out, out_lse,
                           ws_attn, T, s);
  return hip_status(e);
}

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];   // device address of `scratch` per device, once looked up
std::mutex g_scratch_mu;

// Device address of the static scratch on the current device: looked up with
// hipGetSymbolAddress on the first call on that device, then kept.
qsa_status_t scratch_on_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return QSA_ERR_UNSUPPORTED;
  void* p = __atomic_load_n(&g_scratch[dev], __ATOMIC_ACQUIRE);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev];
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_status(e);
      if (p == nullptr) return QSA_ERR_HIP;
      __atomic_store_n(&g_scratch[dev], p, __ATOMIC_RELEASE);
    }
  }
  *out = p;
  return QSA_OK;
}

}  // namespace

qsa_status_t qsa_decode_noalloc(const void* q, const int8_t* q_idx, const int8_t* idx_cache, const void* k_cache,
                                const void* v_cache, const int32_t* page_table, const int32_t* context_lens, int B,
                                int Hq, int Hkv, int head_dim, int n_idx_heads, int idx_dim, int page_size,
                                int max_pages_per_seq, int max_blocks, int k, int P, float softmax_scale,
                                int32_t* block_scores, int32_t* sel_blocks, int32_t* sel_count, float* partial_out,
                                float* partial_lse, float* out, float* out_lse, void* stream) {
  if (B < 0) return QSA_ERR_SHAPE;
  if (B == 0) return QSA_OK;
  // Argument checks first (the size query below assumes sane shapes); a call that fails them
  // returns the same code as qsa_decode, before the scratch is looked up.
  qsa_status_t st = check_index(q_idx, idx_cache, page_table, context_lens, B, n_idx_heads, idx_dim, page_size,
                                max_pages_per_seq, max_blocks, block_scores);
  if (st == QSA_OK) st = check_topk(block_scores, context_lens, B, max_blocks, k, sel_blocks, sel_count);
  if (st == QSA_OK)
    st = check_attn(q, k_cache, v_cache, page_table, context_lens, sel_blocks, sel_count, B, Hq, Hkv, head_dim,
                    page_size, max_pages_per_seq, k, P, partial_out, partial_lse);
  if (st == QSA_OK) st = check_merge(partial_out, partial_lse, B, P, Hq, head_dim, out);
  if (st != QSA_OK) return st;
  const size_t need = qsa_decode_workspace_size(B, Hq, Hkv, max_blocks, k, P);
  if (need > QSA_NOALLOC_SCRATCH_BYTES) return QSA_ERR_SCRATCH;
  void* ws = nullptr;
  if ((st = scratch_on_current_device(&ws)) != QSA_OK) return st;
  return decode_chain(q, q_idx, idx_cache, nullptr, k_cache, v_cache, page_table, context_lens, B, 1, Hq, Hkv,
                      head_dim, n_idx_heads, idx_dim, page_size, max_pages_per_seq, max_blocks, k, P, softmax_scale,
                      block_scores, sel_blocks, sel_count, partial_out, partial_lse, out, out_lse, ws,
                      QSA_NOALLOC_SCRATCH_BYTES, stream);
}

qsa_status_t qsa_decode(const void* q, const int8_t* q_idx, const int8_t* idx_cache, const void* k_cache,
                        const void* v_cache, const int32_t* page_table, const int32_t* context_lens, int B,
                        int Hq, int Hkv, int head_dim, int n_idx_heads, int idx_dim, int page_size,
                        int max_pages_per_seq, int max_blocks, int k, int P, float softmax_scale,
                        int32_t* block_scores, int32_t* sel_blocks, int32_t* sel_count, float* partial_out,
                        float* partial_lse, float* out, float* out_lse, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return decode_chain(q, q_idx, idx_cache, nullptr, k_cache, v_cache, page_table, context_lens, B, 1, Hq, Hkv,
                      head_dim, n_idx_heads, idx_dim, page_size, max_pages_per_seq, max_blocks, k, P, softmax_scale,
                      block_scores, sel_blocks, sel_count, partial_out, partial_lse, out, out_lse, workspace,
                      workspace_bytes, stream);
}

qsa_status_t qsa_decode_pooled(const void* q, const int8_t* q_idx, const int16_t* pooled_cache, const void* k_cache,
                               const void* v_cache, const int32_t* page_table, const int32_t* context_lens, int B,
                               int Hq, int Hkv, int head_dim, int n_idx_heads, int idx_dim, int page_size,
                               int max_pages_per_seq, int max_blocks, int k, int P, float softmax_scale,
                               int32_t* block_scores, int32_t* sel_blocks, int32_t* sel_count, float* partial_out,
                               float* partial_lse, float* out, float* out_lse, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (B > 0 && !pooled_cache) return QSA_ERR_NULL;
  return decode_chain(q, q_idx, nullptr, pooled_cache, k_cache, v_cache, page_table, context_lens, B, 1, Hq, Hkv,
                      head_dim, n_idx_heads, idx_dim, page_size, max_pages_per_seq, max_blocks, k, P, softmax_scale,
                      block_scores, sel_blocks, sel_count, partial_out, partial_lse, out, out_lse, workspace,
                      workspace_bytes, stream);
}

qsa_status_t qsa_index_score_multi(const int8_t* q_idx, const int8_t* idx_cache, const int32_t* page_table,
                                   const int32_t* context_lens, int B, int T, int n_idx_heads, int idx_dim,
                                   int page_size, int max_pages_per_seq, int max_blocks, int32_t* block_scores,
                                   int32_t* page_max, void* stream) {
  if (T < 1) return QSA_ERR_SHAPE;
  if (T > kMaxQueries || (long long)B * T > 65535) return QSA_ERR_UNSUPPORTED;
  qsa_status_t st = check_index(q_idx, idx_cache, page_table, context_lens, B, n_idx_heads, idx_dim, page_size,
                                max_pages_per_seq, max_blocks, block_scores);
  if (st != QSA_OK || B == 0) return st;
  if (max_blocks % 4 != 0 || misaligned(block_scores)) return QSA_ERR_SHAPE;   // 16-byte score stores
  return hip_status(launch_multi_scan(q_idx, idx_cache, page_table, context_lens, B, max_pages_per_seq,
                                      max_blocks, block_scores, page_max, T, (hipStream_t)stream));
}

size_t qsa_decode_multi_workspace_size(int B, int T, int Hq, int Hkv, int max_blocks, int k, int P) {
  if (B <= 0 || T <= 0 || T > kMaxQueries) return 0;
  return qsa_decode_workspace_size(B * T, Hq, Hkv, max_blocks, k, P);
}

qsa_status_t qsa_decode_multi(const void* q, const int8_t* q_idx, const int8_t* idx_cache, const void* k_cache,
                              const void* v_cache, const int32_t* page_table, const int32_t* context_lens, int B,
                              int T, int Hq, int Hkv, int head_dim, int n_idx_heads, int idx_dim, int page_size,
                              int max_pages_per_seq, int max_blocks, int k, int P, float softmax_scale,
                              int32_t* block_scores, int32_t* sel_blocks, int32_t* sel_count, float* partial_out,
                              float* partial_lse, float* out, float* out_lse, void* workspace,
                              size_t workspace_bytes, void* stream) {
  if (B > 0 && T > 0 && (long long)B * T > 65535) return QSA_ERR_UNSUPPORTED;
  return decode_chain(q, q_idx, idx_cache, nullptr, k_cache, v_cache, page_table, context_lens, B, T, Hq, Hkv,
                      head_dim, n_idx_heads, idx_dim, page_size, max_pages_per_seq, max_blocks, k, P, softmax_scale,
                      block_scores, sel_blocks, sel_count, partial_out, partial_lse, out, out_lse, workspace,
                      workspace_bytes, stream);
}

qsa_status_t qsa_decode_multi_pooled(const void* q, const int8_t* q_idx, const int8_t* idx_cache,
                                     const int16_t* pooled_cache, const void* k_cache, const void* v_cache,
                                     const int32_t* page_table, const int32_t* context_lens, int B, int T, int Hq,
                                     int Hkv, int head_dim, int n_idx_heads, int idx_dim, int page_size,
                                     int max_pages_per_seq, int max_blocks, int k, int P, float softmax_scale,
                                     int32_t* block_scores, int32_t* sel_blocks, int32_t* sel_count,
                                     float* partial_out, float* partial_lse, float* out, float* out_lse,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  if (B > 0 && (!pooled_cache || !idx_cache)) return QSA_ERR_NULL;
  if (B > 0 && T > 0 && (long long)B * T > 65535) return QSA_ERR_UNSUPPORTED;
  return decode_chain(q, q_idx, idx_cache, pooled_cache, k_cache, v_cache, page_table, context_lens, B, T, Hq, Hkv,
                      head_dim, n_idx_heads, idx_dim, page_size, max_pages_per_seq, max_blocks, k, P, softmax_scale,
                      block_scores, sel_blocks, sel_count, partial_out, partial_lse, out, out_lse, workspace,
                      workspace_bytes, stream);
}

qsa_status_t qsa_decode_step_pooled(const void* k_new, const void* v_new, const int8_t* idx_new, const int32_t* write,
                                    void* k_cache, void* v_cache, int8_t* idx_cache, int16_t* pooled_cache,
                                    const void* q, const int8_t* q_idx, const int32_t* page_table,
                                    const int32_t* context_lens, int B, int Hq, int Hkv, int head_dim,
                                    int n_idx_heads, int idx_dim, int page_size, int max_pages_per_seq,
                                    int max_blocks, int k, int P, float softmax_scale, int32_t* block_scores,
                                    int32_t* sel_blocks, int32_t* sel_count, float* partial_out, float* partial_lse,
                                    float* out, float* out_lse, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  if (B > 0 && (!k_new || !v_new || !idx_new || !idx_cache || !pooled_cache)) return QSA_ERR_NULL;
  if (B > 0 && (misaligned(k_new) || misaligned(v_new) || misaligned(idx_new) || misaligned(pooled_cache)))
    return QSA_ERR_SHAPE;
  if (Hkv > 64) return QSA_ERR_UNSUPPORTED;
  const StepIn step{k_new, v_new, idx_new, write, k_cache, v_cache, idx_cache};
  return decode_chain(q, q_idx, nullptr, pooled_cache, k_cache, v_cache, page_table, context_lens, B, 1, Hq, Hkv,
                      head_dim, n_idx_heads, idx_dim, page_size, max_pages_per_seq, max_blocks, k, P, softmax_scale,
                      block_scores, sel_blocks, sel_count, partial_out, partial_lse, out, out_lse, workspace,
                      workspace_bytes, stream, &step);
}

qsa_status_t qsa_pool_build(const int8_t* idx_cache, const int32_t* page_table, const int32_t* context_lens, int B,
                            int n_idx_heads, int idx_dim, int page_size, int max_pages_per_seq,
                            int16_t* pooled_cache, void* stream) {
  if (B < 0 || max_pages_per_seq < 1) return QSA_ERR_SHAPE;
  if (n_idx_heads != kIdxHeads || idx_dim != kIdxDim || page_size != kPageSize) return QSA_ERR_UNSUPPORTED;
  if (B > 65535) return QSA_ERR_UNSUPPORTED;
  if (B == 0) return QSA_OK;
  if (!idx_cache || !page_table || !context_lens || !pooled_cache) return QSA_ERR_NULL;
  if (misaligned(idx_cache) || misaligned(pooled_cache)) return QSA_ERR_SHAPE;
  return hip_status(launch_pool_build(idx_cache, page_table, context_lens, B, max_pages_per_seq, pooled_cache,
                                      (hipStream_t)stream));
}

qsa_status_t qsa_cache_append(const void* k_new, const void* v_new, const int8_t* idx_new, const int32_t* write,
                              void* k_cache, void* v_cache, int8_t* idx_cache, int16_t* pooled_cache,
                              const int32_t* page_table, const int32_t* context_lens, int B, int Hkv, int head_dim,
                              int n_idx_heads, int idx_dim, int page_size, int max_pages_per_seq, void* stream) {
  if (B < 0 || Hkv < 1 || max_pages_per_seq < 1) return QSA_ERR_SHAPE;
  if (head_dim != kHeadDim || n_idx_heads != kIdxHeads || idx_dim != kIdxDim || page_size != kPageSize)
    return QSA_ERR_UNSUPPORTED;
  if (B > 65535 || Hkv > 64) return QSA_ERR_UNSUPPORTED;
  if (B == 0) return QSA_OK;
  if (!k_new || !v_new || !idx_new || !k_cache || !v_cache || !idx_cache || !page_table || !context_lens)
    return QSA_ERR_NULL;
  if (misaligned(k_new) || misaligned(v_new) || misaligned(k_cache) || misaligned(v_cache) ||
      misaligned(idx_cache) || (pooled_cache && misaligned(pooled_cache)))
    return QSA_ERR_SHAPE;
  return hip_status(launch_cache_append(k_new, v_new, idx_new, write, k_cache, v_cache, idx_cache, pooled_cache,
                                        page_table, context_lens, B, Hkv, max_pages_per_seq, (hipStream_t)stream));
}

qsa_status_t qsa_index_score_pooled(const int8_t* q_idx, const int16_t* pooled_cache, const int32_t* page_table,
                                    const int32_t* context_lens, int B, int n_idx_heads, int idx_dim, int page_size,
                                    int max_pages_per_seq, int max_blocks, int32_t* block_scores, int32_t* page_max,
                                    void* stream) {
  qsa_status_t st = check_index(q_idx, reinterpret_cast<const int8_t*>(pooled_cache), page_table, context_lens, B,
                                n_idx_heads, idx_dim, page_size, max_pages_per_seq, max_blocks, block_scores);
  if (st != QSA_OK || B == 0) return st;
  return hip_status(launch_index_score_pooled(q_idx, pooled_cache, page_table, context_lens, B, max_pages_per_seq,
                                              max_blocks, block_scores, page_max, nullptr, nullptr, nullptr, nullptr,
                                              nullptr, nullptr, nullptr, 0, (hipStream_t)stream, 1, nullptr));
}

qsa_status_t qsa_check_pages(const int32_t* page_table, const int32_t* context_lens, int B,
                             int max_pages_per_seq, int page_size, int num_pages, int32_t* verdict,
                             void* stream) {
  if (B < 0 || max_pages_per_seq < 1 || page_size < 1 || num_pages < 0) return QSA_ERR_SHAPE;
  if (B > 65535) return QSA_ERR_UNSUPPORTED;
  if (B == 0) return QSA_OK;
  if (!page_table || !context_lens || !verdict) return QSA_ERR_NULL;
  return hip_status(launch_check_pages(page_table, context_lens, B, max_pages_per_seq, page_size, num_pages,
                                       verdict, (hipStream_t)stream));
}

qsa_status_t qsa_workspace_clear(void* workspace, size_t workspace_bytes, void* stream) {
  if (workspace_bytes == 0) return QSA_OK;
  if (!workspace) return QSA_ERR_NULL;
  if ((workspace_bytes & 3u) != 0 || misaligned(workspace)) return QSA_ERR_SHAPE;
  const size_t nwords = workspace_bytes / 4;
  size_t grid = (nwords + 255) / 256;
  if (grid > 4096) grid = 4096;
  hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream,
                     static_cast<uint32_t*>(workspace), nwords);
  return hip_status(hipGetLastError());
}

}  // extern "C"
