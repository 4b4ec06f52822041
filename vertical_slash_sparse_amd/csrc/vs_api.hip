// vs_api.hip -- the C ABI of libvs (declared in include/vs.h): argument
// checks, workspace sizing, launches.  Everything that can be checked on the
// host is checked before anything is enqueued; nothing here allocates,
// frees or synchronises except vs_attn_tile_counts, which reads counters back.
#include <limits.h>
#include <math.h>

#include <mutex>

#include "vs.h"
#include "vs_internal.h"

using namespace vs;

// Device memory for callers that cannot allocate: the workspace of
// vs_sparse_attn_prefill_noalloc.  Every GPU the library runs on holds its
// own copy until the process ends.  Host code never names the array
// directly (on the host the name is only a stand-in): each device's address
// comes from hipGetSymbolAddress, taken once per device.
static __device__ __align__(256) uint8_t scratch[VS_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// the current device's copy of `scratch` (null if it cannot be had)
void* scratch_of_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

bool group_ok(int h_q, int h_kv) {
  if (h_q <= 0 || h_kv <= 0 || h_q % h_kv) return false;
  const int g = h_q / h_kv;
  return g == 1 || g == 2 || g == 4 || g == 8 || g == 16;
}

vs_status from_hip(hipError_t e) { return e == hipSuccess ? VS_OK : VS_ERR_HIP; }

// a launch of `wgs` workgroups of `threads` work-items fits one grid dimension
bool grid_fits(long long wgs, int threads) { return wgs >= 0 && wgs * threads < kGridItems; }

// The tile builder runs one workgroup per index-set row, and the attention
// kernel one per (row, query block); both grids must fit.
vs_status attn_grid_status(int group, int rows, long long n) {
  if (!grid_fits(rows, kBuildThreads)) return VS_ERR_UNSUPPORTED;
  if (!grid_fits(attn_workgroups(group, rows, n), kAttnThreads)) return VS_ERR_UNSUPPORTED;
  return VS_OK;
}

}  // namespace

extern "C" {

const char* vs_status_str(vs_status s) {
  switch (s) {
    case VS_OK: return "ok";
    case VS_ERR_INVALID: return "invalid argument";
    case VS_ERR_UNSUPPORTED: return "unsupported shape";
    case VS_ERR_WORKSPACE: return "workspace too small";
    case VS_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

vs_status vs_index(const void* k_rope, const void* v, int h_kv, int n, int d, int hidden,
                   const void* w1, const void* w2, float* vlog, float* slog,
                   hipStream_t stream) {
  if (!k_rope || !v || !w1 || !w2 || !vlog || !slog) return VS_ERR_INVALID;
  if (h_kv <= 0 || n <= 0 || d <= 0 || hidden <= 0) return VS_ERR_INVALID;
  if ((long long)h_kv * n > (1LL << 40)) return VS_ERR_INVALID;
  if ((d != 64 && d != 128) || hidden % 32 || hidden > kIdxMaxHidden) return VS_ERR_UNSUPPORTED;
  // K and V are each read through one buffer resource with a 32-bit range
  if ((long long)h_kv * n * d * 2 >= (1LL << 32)) return VS_ERR_UNSUPPORTED;
  return from_hip(launch_index(k_rope, v, h_kv, n, d, hidden, w1, w2, vlog, slog, stream));
}

size_t vs_select_workspace_bytes(int heads, int n) {
  if (heads <= 0 || n <= 0) return 0;
  return SelectWsLayout(heads, n).total;
}

vs_status vs_select(const float* logit, int heads, int n, vs_kind kind, double mass, int cap,
                    int32_t* idx, int32_t* count, void* ws, size_t ws_bytes,
                    hipStream_t stream) {
  if (!logit || !idx || !count || !ws) return VS_ERR_INVALID;
  if (heads <= 0 || n <= 0 || heads > 65535) return VS_ERR_INVALID;
  if (kind != VS_VERTICAL && kind != VS_SLASH) return VS_ERR_INVALID;
  if (!(mass > 0.0 && mass <= 1.0)) return VS_ERR_INVALID;
  if (cap < 1 || cap > n) return VS_ERR_INVALID;
  if (ws_bytes < vs_select_workspace_bytes(heads, n)) return VS_ERR_WORKSPACE;
  return from_hip(launch_select(logit, heads, n, (int)kind, mass, 0ull, cap, idx, count, ws, stream));
}

size_t vs_select_both_workspace_bytes(int heads, int n) {
  if (heads <= 0 || n <= 0 || heads > 32767) return 0;
  return SelectWsLayout(2 * heads, n).total;
}

vs_status vs_select_both(const float* vlog, const float* slog, int heads, int n, double mass,
                         int cap_v, int cap_s, int32_t* v_idx, int32_t* v_cnt, int32_t* s_off,
                         int32_t* s_cnt, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!vlog || !slog || !v_idx || !v_cnt || !s_off || !s_cnt || !ws) return VS_ERR_INVALID;
  if (heads <= 0 || n <= 0 || heads > 32767) return VS_ERR_INVALID;
  if (!(mass > 0.0 && mass <= 1.0)) return VS_ERR_INVALID;
  if (cap_v < 1 || cap_v > n || cap_s < 1 || cap_s > n) return VS_ERR_INVALID;
  if (ws_bytes < vs_select_both_workspace_bytes(heads, n)) return VS_ERR_WORKSPACE;
  const SelSide sides[2] = {{vlog, v_idx, v_cnt, (int)VS_VERTICAL, cap_v},
                            {slog, s_off, s_cnt, (int)VS_SLASH, cap_s}};
  return from_hip(launch_select_sides(sides, 2, heads, n, mass, 0ull, ws, stream));
}

vs_status vs_select_threshold(const float* logit, int heads, int n, vs_kind kind, double alpha,
                              int cap, int32_t* idx, int32_t* count, void* ws, size_t ws_bytes,
                              hipStream_t stream) {
  if (!logit || !idx || !count || !ws) return VS_ERR_INVALID;
  if (heads <= 0 || n <= 0 || heads > 65535) return VS_ERR_INVALID;
  if (kind != VS_VERTICAL && kind != VS_SLASH) return VS_ERR_INVALID;
  if (!(alpha > 0.0 && alpha <= 1.0)) return VS_ERR_INVALID;
  if (cap < 1 || cap > n) return VS_ERR_INVALID;
  if (ws_bytes < vs_select_workspace_bytes(heads, n)) return VS_ERR_WORKSPACE;
  const unsigned long long thresh = (unsigned long long)ceil(alpha * 4294967296.0);
  return from_hip(launch_select(logit, heads, n, (int)kind, 1.0, thresh, cap, idx, count, ws, stream));
}

size_t vs_attn_workspace_bytes(int h_kv, int n, int cap_v, int cap_s) {
  if (h_kv <= 0 || n <= 0 || cap_v < 1 || cap_s < 1) return 0;
  return AttnWsLayout(h_kv, n, cap_v, cap_s).total;
}

vs_status vs_sparse_attn_prefill(const void* q, const void* k, const void* v, vs_dtype dt,
                                 int h_q, int h_kv, int n, int d, float scale,
                                 const int32_t* v_idx, const int32_t* v_cnt, int cap_v,
                                 const int32_t* s_off, const int32_t* s_cnt, int cap_s,
                                 void* out, float* lse, void* ws, size_t ws_bytes,
                                 hipStream_t stream) {
  if (!q || !k || !v || !v_idx || !v_cnt || !s_off || !s_cnt || !out || !ws) return VS_ERR_INVALID;
  if (dt != VS_BF16 && dt != VS_F32) return VS_ERR_INVALID;
  if (h_q <= 0 || h_kv <= 0 || n <= 0 || d <= 0) return VS_ERR_INVALID;
  if (h_q % h_kv) return VS_ERR_INVALID;
  if (cap_v < 1 || cap_s < 1) return VS_ERR_INVALID;
  if (!isfinite(scale)) return VS_ERR_INVALID;
  if ((long long)n > (1LL << 30) || (long long)h_kv * n * d > (1LL << 40)) return VS_ERR_INVALID;
  if (!group_ok(h_q, h_kv)) return VS_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return VS_ERR_UNSUPPORTED;
  // one KV head must fit a 32-bit buffer range
  if ((long long)n * d * (dt == VS_F32 ? 4 : 2) >= (1LL << 31)) return VS_ERR_UNSUPPORTED;
  if (attn_grid_status(h_q / h_kv, h_kv, n) != VS_OK) return VS_ERR_UNSUPPORTED;
  if (ws_bytes < vs_attn_workspace_bytes(h_kv, n, cap_v, cap_s)) return VS_ERR_WORKSPACE;
  return from_hip(launch_attn(q, k, v, dt == VS_F32, h_q, h_kv, n, d, scale, v_idx, v_cnt, cap_v,
                              s_off, s_cnt, cap_s, out, lse, ws, stream));
}

vs_status vs_sparse_attn_prefill_noalloc(const void* q, const void* k, const void* v, vs_dtype dt,
                                         int h_q, int h_kv, int n, int d, float scale,
                                         const int32_t* v_idx, const int32_t* v_cnt, int cap_v,
                                         const int32_t* s_off, const int32_t* s_cnt, int cap_s,
                                         void* out, float* lse, hipStream_t stream) {
  // the same checks as vs_sparse_attn_prefill, with the static scratch as the
  // workspace; sizes past it are rejected before anything is launched
  if (!q || !k || !v || !v_idx || !v_cnt || !s_off || !s_cnt || !out) return VS_ERR_INVALID;
  if (h_q <= 0 || h_kv <= 0 || n <= 0 || cap_v < 1 || cap_s < 1) return VS_ERR_INVALID;
  if (vs_attn_workspace_bytes(h_kv, n, cap_v, cap_s) > (size_t)VS_NOALLOC_SCRATCH_BYTES)
    return VS_ERR_WORKSPACE;
  void* ws = scratch_of_current_device();
  if (!ws) return VS_ERR_HIP;
  return vs_sparse_attn_prefill(q, k, v, dt, h_q, h_kv, n, d, scale, v_idx, v_cnt, cap_v, s_off,
                                s_cnt, cap_s, out, lse, ws, (size_t)VS_NOALLOC_SCRATCH_BYTES,
                                stream);
}

namespace {

// checks shared by the per-query-head and packed-batch forms
vs_status check_attn_common(const void* q, const void* k, const void* v, vs_dtype dt, int h_q,
                            int h_kv, int d, float scale, int cap_v, int cap_s, const void* out,
                            const void* ws) {
  if (!q || !k || !v || !out || !ws) return VS_ERR_INVALID;
  if (dt != VS_BF16 && dt != VS_F32) return VS_ERR_INVALID;
  if (h_q <= 0 || h_kv <= 0 || d <= 0 || h_q % h_kv) return VS_ERR_INVALID;
  if (cap_v < 1 || cap_s < 1) return VS_ERR_INVALID;
  if (!isfinite(scale)) return VS_ERR_INVALID;
  if (!group_ok(h_q, h_kv)) return VS_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return VS_ERR_UNSUPPORTED;
  return VS_OK;
}

}  // namespace

vs_status vs_sparse_attn_prefill_qh(const void* q, const void* k, const void* v, vs_dtype dt,
                                    int h_q, int h_kv, int n, int d, float scale,
                                    const int32_t* v_idx, const int32_t* v_cnt, int cap_v,
                                    const int32_t* s_off, const int32_t* s_cnt, int cap_s,
                                    void* out, float* lse, void* ws, size_t ws_bytes,
                                    hipStream_t stream) {
  if (!v_idx || !v_cnt || !s_off || !s_cnt) return VS_ERR_INVALID;
  const vs_status st = check_attn_common(q, k, v, dt, h_q, h_kv, d, scale, cap_v, cap_s, out, ws);
  if (st != VS_OK) return st;
  if (n <= 0 || (long long)n > (1LL << 30) || (long long)h_q * n * d > (1LL << 40)) return VS_ERR_INVALID;
  if ((long long)n * d * (dt == VS_F32 ? 4 : 2) >= (1LL << 31)) return VS_ERR_UNSUPPORTED;
  if (attn_grid_status(1, h_q, n) != VS_OK) return VS_ERR_UNSUPPORTED;
  if (ws_bytes < vs_attn_workspace_bytes(h_q, n, cap_v, cap_s)) return VS_ERR_WORKSPACE;
  AttnLayout lay;
  lay.kvdiv = h_q / h_kv;
  return from_hip(launch_attn(q, k, v, dt == VS_F32, h_q, h_q, n, d, scale, v_idx, v_cnt, cap_v,
                              s_off, s_cnt, cap_s, out, lse, ws, stream, lay));
}

vs_status vs_sparse_attn_prefill_varlen(const void* q, const void* k, const void* v, vs_dtype dt,
                                        int h_q, int h_kv, int total_n, int d, float scale,
                                        const int32_t* cu_seqlens, int nseq,
                                        int sets_per_query_head, const int32_t* v_idx,
                                        const int32_t* v_cnt, int cap_v, const int32_t* s_off,
                                        const int32_t* s_cnt, int cap_s, void* out, float* lse,
                                        void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!cu_seqlens || !v_idx || !v_cnt || !s_off || !s_cnt) return VS_ERR_INVALID;
  const vs_status st = check_attn_common(q, k, v, dt, h_q, h_kv, d, scale, cap_v, cap_s, out, ws);
  if (st != VS_OK) return st;
  if (nseq <= 0 || total_n <= 0 || (long long)h_q * total_n * d > (1LL << 40)) return VS_ERR_INVALID;
  if (cu_seqlens[0] != 0 || cu_seqlens[nseq] != total_n) return VS_ERR_INVALID;
  const int sets = sets_per_query_head ? h_q : h_kv;
  const int group = h_q / sets;
  int max_len = 0;
  long long wgs = 0;
  for (int s = 0; s < nseq; ++s) {
    const int len = cu_seqlens[s + 1] - cu_seqlens[s];
    if (len < 0) return VS_ERR_INVALID;
    if (len > max_len) max_len = len;
    wgs += attn_workgroups(group, sets, len);
  }
  if ((long long)max_len * d * (dt == VS_F32 ? 4 : 2) >= (1LL << 31)) return VS_ERR_UNSUPPORTED;
  if ((long long)nseq * sets > INT_MAX / 2) return VS_ERR_UNSUPPORTED;
  if (!grid_fits((long long)nseq * sets, kBuildThreads) || !grid_fits(wgs, kAttnThreads))
    return VS_ERR_UNSUPPORTED;
  if (ws_bytes < vs_attn_varlen_workspace_bytes(sets, nseq, max_len, cap_v, cap_s))
    return VS_ERR_WORKSPACE;
  return from_hip(launch_attn_varlen(q, k, v, dt == VS_F32, h_q, sets,
                                     sets_per_query_head ? h_q / h_kv : 1, total_n, d, scale,
                                     cu_seqlens, nseq, max_len, v_idx, v_cnt, cap_v, s_off, s_cnt,
                                     cap_s, out, lse, ws, stream));
}

size_t vs_attn_varlen_workspace_bytes(int sets, int nseq, int max_len, int cap_v, int cap_s) {
  if (sets <= 0 || nseq <= 0 || max_len < 0 || cap_v < 1 || cap_s < 1) return 0;
  if ((long long)nseq * sets > INT_MAX / 2) return 0;
  return AttnWsLayout(nseq * sets, max_len, cap_v, cap_s, attn_varlen_table_ints(nseq)).total;
}

size_t vs_aggregate_workspace_bytes(int h_kv, int n) {
  if (h_kv <= 0 || n <= 0) return 0;
  return aggregate_workspace_bytes(h_kv, n);
}

vs_status vs_attn_aggregate(const void* q, const void* k, const void* v, int h_q, int h_kv, int n,
                            int d, float scale, void* out, float* lse, float* a_v, float* a_s,
                            void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!q || !k || !v || !out || !lse || !a_v || !a_s || !ws) return VS_ERR_INVALID;
  if (h_q <= 0 || h_kv <= 0 || n <= 0 || d <= 0 || h_q % h_kv) return VS_ERR_INVALID;
  if (!isfinite(scale)) return VS_ERR_INVALID;
  if ((long long)n > (1LL << 30) || (long long)h_kv * n * d > (1LL << 40)) return VS_ERR_INVALID;
  if (!group_ok(h_q, h_kv)) return VS_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return VS_ERR_UNSUPPORTED;
  if ((long long)n * d * 2 >= (1LL << 31)) return VS_ERR_UNSUPPORTED;
  if (h_kv > 65535 || !aggregate_grid_fits(h_q, h_kv, n)) return VS_ERR_UNSUPPORTED;
  if (attn_grid_status(h_q / h_kv, h_kv, n) != VS_OK) return VS_ERR_UNSUPPORTED;
  if (ws_bytes < vs_aggregate_workspace_bytes(h_kv, n)) return VS_ERR_WORKSPACE;
  return from_hip(launch_aggregate(q, k, v, h_q, h_kv, n, d, scale, out, lse, a_v, a_s, ws, stream));
}

size_t vs_block_workspace_bytes(int h_kv, int n, int d) {
  if (h_kv <= 0 || n <= 0 || d <= 0) return 0;
  return block_workspace_bytes(h_kv, n, d);
}

vs_status vs_block_discover(const void* q, const void* k, int h_q, int h_kv, int n, int d,
                            float scale, int skel, float alpha, uint32_t* mask, int words_per_row,
                            float* score, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!q || !k || !mask || !ws) return VS_ERR_INVALID;
  if (h_q <= 0 || h_kv <= 0 || n <= 0 || d <= 0 || h_q % h_kv) return VS_ERR_INVALID;
  if (!isfinite(scale)) return VS_ERR_INVALID;
  if (!(alpha > 0.f && alpha <= 1.f)) return VS_ERR_INVALID;
  if (skel < 1 || skel > kBN || kBN % skel) return VS_ERR_INVALID;
  if ((long long)n > (1LL << 30) || (long long)h_q * n * d > (1LL << 40)) return VS_ERR_INVALID;
  const long long nb = ((long long)n + kBN - 1) / kBN;
  if ((long long)words_per_row * 32 < nb) return VS_ERR_INVALID;
  if (!group_ok(h_q, h_kv)) return VS_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return VS_ERR_UNSUPPORTED;
  if ((h_q / h_kv) * skel > 32) return VS_ERR_UNSUPPORTED;
  if (nb > kBlkMaxBlocks) return VS_ERR_UNSUPPORTED;
  if (h_kv > 65535 || !block_discover_grid_fits(h_kv, n)) return VS_ERR_UNSUPPORTED;
  if (ws_bytes < vs_block_workspace_bytes(h_kv, n, d)) return VS_ERR_WORKSPACE;
  return from_hip(launch_block_discover(q, k, h_q, h_kv, n, d, scale, skel, alpha, mask,
                                        words_per_row, score, ws, stream));
}

size_t vs_block_attn_workspace_bytes(void) { return 256; }

vs_status vs_block_attn_prefill(const void* q, const void* k, const void* v, vs_dtype dt, int h_q,
                                int h_kv, int n, int d, float scale, const uint32_t* mask,
                                int words_per_row, void* out, float* lse, void* ws,
                                size_t ws_bytes, hipStream_t stream) {
  if (!q || !k || !v || !mask || !out || !ws) return VS_ERR_INVALID;
  if (dt != VS_BF16 && dt != VS_F32) return VS_ERR_INVALID;
  if (h_q <= 0 || h_kv <= 0 || n <= 0 || d <= 0 || h_q % h_kv) return VS_ERR_INVALID;
  if (!isfinite(scale)) return VS_ERR_INVALID;
  // block indices travel in 24 bits beside per-query-block flags
  if ((long long)n > (1LL << 30) - kBN || (long long)h_kv * n * d > (1LL << 40)) return VS_ERR_INVALID;
  const long long nb = ((long long)n + kBN - 1) / kBN;
  if ((long long)words_per_row * 32 < nb) return VS_ERR_INVALID;
  if (!group_ok(h_q, h_kv)) return VS_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return VS_ERR_UNSUPPORTED;
  if ((long long)n * d * (dt == VS_F32 ? 4 : 2) >= (1LL << 31)) return VS_ERR_UNSUPPORTED;
  if (!grid_fits(attn_workgroups(h_q / h_kv, h_kv, n), kAttnThreads)) return VS_ERR_UNSUPPORTED;
  if (ws_bytes < vs_block_attn_workspace_bytes()) return VS_ERR_WORKSPACE;
  return from_hip(launch_attn_blocks(q, k, v, dt == VS_F32, h_q, h_kv, n, d, scale, mask,
                                     words_per_row, out, lse, ws, stream));
}

vs_status vs_attn_tile_counts(const void* ws, int h_kv, int n, int cap_v, int cap_s, int h_q,
                              int64_t tiles[4], hipStream_t stream) {
  if (!ws || !tiles) return VS_ERR_INVALID;
  if (h_kv <= 0 || n <= 0 || cap_v < 1 || cap_s < 1) return VS_ERR_INVALID;
  if (!group_ok(h_q, h_kv)) return VS_ERR_UNSUPPORTED;
  const AttnWsLayout L(h_kv, n, cap_v, cap_s);
  unsigned long long host[2] = {0ull, 0ull};
  hipError_t e = hipMemcpyAsync(host, static_cast<const char*>(ws) + L.off_stats, sizeof host,
                                hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return VS_ERR_HIP;
  const int group = h_q / h_kv;
  tiles[0] = (int64_t)host[0];
  tiles[1] = (int64_t)host[1];
  tiles[2] = (int64_t)attn_query_rows_per_block(group);
  tiles[3] = (int64_t)kBN;
  return VS_OK;
}

}  // extern "C"
