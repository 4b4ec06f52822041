// vs_internal.h -- launch entry points and workspace layouts shared between
// the C-ABI shim (vs_api.hip) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace vs {

constexpr int kBN = 64;          // keys per attention tile
constexpr int kPrePad = 4;       // zero words before each bitmap (windows may start below 0)
constexpr int kPostPad = 8;      // zero words after each bitmap (windows may run past n)
constexpr int kListCap = 2048;   // LDS list of gathered columns per refill
// u64 words of an attention call's counters: tile counts [0, 2), unused
// [2, 4), the work-item queues (8 u32) [4, 8)
constexpr int kStatWords = 8;

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Device workspace of vs_sparse_attn_prefill, per call.
struct AttnWsLayout {
  int words;        // bitmap words covering positions [0, n)
  int stride;       // words per head in a bitmap array (pads included)
  size_t off_bitO, off_bitV, off_prefO, off_cleanO, off_cleanV, off_clLo, off_clHi, off_counts,
      off_stats, off_tab, total;
  // h_kv rows of index sets over positions [0, n); tab_ints more ints hold a
  // packed batch's sequence table
  AttnWsLayout(int h_kv, int n, int cap_v, int cap_s, int tab_ints = 0) {
    words = (n + 31) / 32;
    stride = kPrePad + words + kPostPad;
    size_t o = 0;
    auto take = [&](size_t bytes) { size_t at = o; o = align_up(o + bytes, 256); return at; };
    off_bitO = take(sizeof(uint32_t) * (size_t)h_kv * stride);
    off_bitV = take(sizeof(uint32_t) * (size_t)h_kv * stride);
    off_prefO = take(sizeof(uint32_t) * (size_t)h_kv * (words + 1));
    off_cleanO = take(sizeof(int32_t) * (size_t)h_kv * cap_s);
    off_cleanV = take(sizeof(int32_t) * (size_t)h_kv * cap_v);
    off_clLo = take(sizeof(int32_t) * (size_t)h_kv * cap_s);
    off_clHi = take(sizeof(int32_t) * (size_t)h_kv * cap_s);
    off_counts = take(sizeof(int32_t) * 4 * (size_t)h_kv);
    off_stats = take(sizeof(unsigned long long) * kStatWords);
    off_tab = take(sizeof(int32_t) * (size_t)tab_ints);
    total = o;
  }
};

constexpr int kSelChunk = 8192;     // candidates per selection workgroup
constexpr int kSelStateWords = 32;  // u64 decision-state words per selection row

// Device workspace of vs_select: per row, each chunk's largest key, the
// decision state, one (count, mass) histogram of kSelBins bins per digit pass,
// and each chunk's published counts of candidates above and tied with the
// K-th.
constexpr int kSelBins = 2048;
constexpr int kSelDigitPasses = 3;
struct SelectWsLayout {
  int chunks;  // workgroups per row
  size_t off_cmax, off_state, off_hcnt, off_hmass, off_slot, total;
  SelectWsLayout(int rows, int n) {
    chunks = (n + kSelChunk - 1) / kSelChunk;
    size_t o = 0;
    auto take = [&](size_t bytes) { size_t at = o; o = align_up(o + bytes, 256); return at; };
    off_cmax = take(sizeof(uint32_t) * (size_t)rows * chunks);
    off_state = take(sizeof(uint64_t) * kSelStateWords * (size_t)rows);
    off_hcnt = take(sizeof(uint32_t) * kSelDigitPasses * kSelBins * (size_t)rows);
    off_hmass = take(sizeof(uint64_t) * kSelDigitPasses * kSelBins * (size_t)rows);
    off_slot = take(sizeof(uint64_t) * (size_t)rows * chunks);
    total = o;
  }
};

// Where a call's rows live (see AttnParams): set head g reads K/V head
// g / kvdiv; row r of head h is row h * hstride + row0 + r (hstride 0 = n).
struct AttnLayout {
  int kvdiv = 1;
  long long hstride = 0;
  long long row0 = 0;
  bool full_tiles = false;  // nearly every tile has all its keys selected
};

hipError_t launch_attn(const void* q, const void* k, const void* v, bool f32, int h_q, int h_kv,
                       int n, int d, float scale, const int32_t* v_idx, const int32_t* v_cnt,
                       int cap_v, const int32_t* s_off, const int32_t* s_cnt, int cap_s, void* out,
                       float* lse, void* ws, hipStream_t stream,
                       const AttnLayout& lay = AttnLayout());

// A packed batch (cu_seqlens on the host, nseq + 1 entries) in one tile
// build and one attention launch: sets index-set heads per sequence, lists
// [nseq][sets][cap], workspace AttnWsLayout(nseq * sets, max_len, cap_v,
// cap_s, attn_varlen_table_ints(nseq)).
int attn_varlen_table_ints(int nseq);
hipError_t launch_attn_varlen(const void* q, const void* k, const void* v, bool f32, int h_q,
                              int sets, int kvdiv, int total_n, int d, float scale,
                              const int32_t* cu_seqlens, int nseq, int max_len,
                              const int32_t* v_idx, const int32_t* v_cnt, int cap_v,
                              const int32_t* s_off, const int32_t* s_cnt, int cap_s, void* out,
                              float* lse, void* ws, hipStream_t stream);

int attn_query_rows_per_block(int group);
// workgroups of one attention launch over `sets` index-set rows of n
// positions each (G = group query heads per set)
long long attn_workgroups(int group, int sets, long long n);
constexpr int kAttnThreads = 512;      // threads per attention workgroup
constexpr int kBuildThreads = 1024;    // threads per workgroup of the per-row builder passes
// a launch's work-items along one grid dimension must stay below 2^32
constexpr long long kGridItems = 1LL << 32;

size_t aggregate_workspace_bytes(int h_kv, int n);
// the aggregation's own pass fits one grid dimension
bool aggregate_grid_fits(int h_q, int h_kv, long long n);
// block-sparse mode of the attention kernel: ws holds 32 bytes of counters
hipError_t launch_attn_blocks(const void* q, const void* k, const void* v, bool f32, int h_q,
                              int h_kv, int n, int d, float scale, const uint32_t* blk, int wpr,
                              void* out, float* lse, void* ws, hipStream_t stream);

// FlashPrefill block discovery
constexpr int kBlkMaxBlocks = 16384;  // key blocks a discovery call may have
size_t block_workspace_bytes(int h_kv, int n, int d);
bool block_discover_grid_fits(int h_kv, long long n);
hipError_t launch_block_discover(const void* q, const void* k, int h_q, int h_kv, int n, int d,
                                 float scale, int skel, float alpha, uint32_t* mask, int wpr,
                                 float* score, void* ws, hipStream_t stream);

hipError_t launch_aggregate(const void* q, const void* k, const void* v, int h_q, int h_kv, int n,
                            int d, float scale, void* out, float* lse, float* a_v, float* a_s,
                            void* ws, hipStream_t stream);

// mass in (0, 1] with thresh == 0: cumulative-mass budget; thresh > 0: keep
// quantised masses >= thresh (max-based threshold)
// One kind of candidates of a selection: [heads][n] scores in, [heads][cap]
// indices and [heads] counts out.
struct SelSide {
  const float* logit;
  int32_t* idx;
  int32_t* count;
  int kind, cap;
};
// The selection chain over nsides (1 or 2) kinds at once, each for `heads`
// heads; the workspace holds nsides * heads rows (SelectWsLayout).
hipError_t launch_select_sides(const SelSide* sides, int nsides, int heads, int n, double mass,
                               unsigned long long thresh, void* ws, hipStream_t stream);
hipError_t launch_select(const float* logit, int heads, int n, int kind, double mass,
                         unsigned long long thresh, int cap, int32_t* idx, int32_t* count, void* ws,
                         hipStream_t stream);

// VSIndexer: d in {64, 128}; hidden a multiple of 32 up to kIdxMaxHidden
// (its first-layer weights are held in registers)
constexpr int kIdxMaxHidden = 256;
hipError_t launch_index(const void* k, const void* v, int h_kv, int n, int d, int hidden,
                        const void* w1, const void* w2, float* vlog, float* slog,
                        hipStream_t stream);

}  // namespace vs
