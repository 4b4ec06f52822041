// vs_index.hip -- VSIndexer scoring for gfx950.
//
// VSPrefill (gist.science summaries of arXiv 2603.04460, English page,
// Technical Summary section 2, "Key Components 1. VSIndexer"): a
// shared-weight two-layer linear network over concat(K with RoPE, V) with
// separate down-projection heads for vertical and slash importance:
//     h_j = max(0, W1 [k_j | v_j]),   vlog_j = W2[0] . h_j,   slog_j = W2[1] . h_j.
//
// Each position reads 2*d*2 bytes (512 at d = 128) and costs 2*(2d)*hidden +
// 2*2*hidden flops, about hidden flop per byte (128 at hidden = 128) -- under
// the MI355X ridge (~315 flop/B for bf16 MFMA against 8 TB/s), so the kernel
// is HBM-bound and is built to stream:
//  * a workgroup of four waves takes 32 consecutive positions at a time; their
//    K and V rows (16 KiB at d = 128, contiguous in HBM) arrive by LDS-DMA into
//    a ring of four stages, so every HBM read is a full 1 KiB line run and
//    three blocks are in flight while one is multiplied;
//  * the hidden units come in chunks of 32; wave w owns chunks w, w + 4 (at
//    most two, so hidden <= 256): their slices of W1 (the A operand of
//    H^T = W1 X^T on v_mfma_f32_32x32x16_bf16) and of W2 stay in registers for
//    the whole kernel, and the 32 positions are the B operand, read from LDS;
//  * the second layer runs in fp32 on the vector ALUs from the fp32
//    accumulators; the four waves' partial sums meet in LDS and are added
//    after the next block's barrier, so each block costs one barrier.
#include "vs_common.h"
#include "vs_internal.h"

namespace vs {

namespace {

constexpr int kIdxRows = 32;          // positions per block
constexpr int kIdxNst = 4;            // ring stages
constexpr int kIdxThreads = 256;
constexpr int kIdxWaves = kIdxThreads / 64;

// XOR swizzle of the 16-byte chunks of an LDS row, so that lanes reading one
// chunk of consecutive rows hit distinct banks
template <int D>
__device__ __forceinline__ int idx_swz(int r) {
  if constexpr (D == 128) return ((r & 7) << 1) | ((r >> 3) & 1);
  else return (((r >> 1) & 3) << 1) | ((r >> 3) & 1);
}

// D: head dim (the input is 2D wide); CPW: hidden chunks of 32 per wave
// (nch = hidden / 32 chunks in all, wave w owning chunks w and w + 4)
template <int D, int CPW>
__global__ __launch_bounds__(kIdxThreads, 2) void index_kernel(const uint16_t* __restrict__ k,
                                                               const uint16_t* __restrict__ v,
                                                               const uint16_t* __restrict__ w1,
                                                               const uint16_t* __restrict__ w2,
                                                               float* __restrict__ vlog,
                                                               float* __restrict__ slog,
                                                               long long total_rows, int nch) {
  constexpr int X = 2 * D;                  // indexer input width
  constexpr int KS = X / 16;                // k-steps of the first layer (half on K, half on V)
  constexpr int ROWB = D * 2;               // bytes of one K (or V) row
  constexpr int CH = ROWB / 16;             // 16-byte chunks per row
  constexpr int RPD = 1024 / ROWB;          // rows per 1 KiB DMA
  constexpr int STAGEB = 2 * kIdxRows * ROWB;  // K rows then V rows
  constexpr int KPM = kIdxRows * ROWB / 1024;  // KiB per matrix of a stage
  constexpr int NDMA = 2 * KPM / kIdxWaves;    // 1 KiB loads per wave per block
  static_assert(NDMA >= 1 && NDMA * kIdxWaves == 2 * KPM, "stage split");
  __shared__ __align__(16) uint8_t xs[kIdxNst * STAGEB];
  __shared__ float2 red[2][kIdxWaves][kIdxRows];  // [block parity][wave][position] partial (vertical, slash)
  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  lds_u8* const xbase = (lds_u8*)xs;

  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, ql = lane & 31;
  const int wave = wave_uniform(tid >> 6);
  const int hid = 32 * nch;  // hidden width

  // DMA: wave w moves NDMA KiB of each block; a KiB holds RPD rows, lane l
  // row (l / CH) of them, chunk slot l % CH, which holds source chunk
  // slot ^ swizzle(row)
  const uint32_t rbytes = (uint32_t)(total_rows * ROWB);
  const u32x4 wk = buffer_words(k, rbytes);
  const u32x4 wv = buffer_words(v, rbytes);
  int dma_lds[NDMA], dma_src[NDMA], dma_mat[NDMA];
#pragma unroll
  for (int i = 0; i < NDMA; ++i) {
    const int kib = wave * NDMA + i;   // K rows in KiB 0..KPM-1, V rows in KPM..2KPM-1
    const int mat = kib >= KPM ? 1 : 0;
    const int r = RPD * (kib % KPM) + lane / CH;
    dma_mat[i] = mat;
    dma_lds[i] = kib * 1024;
    dma_src[i] = r * ROWB + 16 * ((lane % CH) ^ idx_swz<D>(r));
  }
  unsigned dma_off[NDMA];
  auto stage_block = [&](long long blk, int st) {
    const unsigned base = (unsigned)(blk * kIdxRows * ROWB);  // past the end: out of range, zeros
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
      const unsigned off = blk * kIdxRows < total_rows ? base + (unsigned)dma_src[i] : rbytes;
      dma16(dma_mat[i] ? wv : wk, (uint32_t)(uintptr_t)(xbase + st * STAGEB + dma_lds[i]), off);
      dma_off[i] = off;
    }
  };
  // B operand (k-step s of one matrix) of a stage: position ql, chunk 2s + half
  int boff[KS / 2];
#pragma unroll
  for (int s = 0; s < KS / 2; ++s) boff[s] = ql * ROWB + 16 * ((2 * s + half) ^ idx_swz<D>(ql));

  const long long nblk = (total_rows + kIdxRows - 1) / kIdxRows;
  const long long first = blockIdx.x, stride = gridDim.x;
  if (first >= nblk) return;
  const long long mine = (nblk - first + stride - 1) / stride;  // blocks of this workgroup
  for (int j = 0; j < kIdxNst - 1; ++j) stage_block(first + j * stride < nblk ? first + j * stride : nblk, j);

  // The first blocks' loads are already in flight: the weights' own latency
  // (they come from L2 or HBM on a call's first use) overlaps them.
  // Chunk c = wave + 4 cc covers hidden units 32 c ..; its W1 rows 32 c + ql
  // are the A operands (k-step s: input dims 16 s + 8 half ..).  A wave past
  // the last chunk holds zeros and skips the products.
  bool has[CPW];
  bf16x8 wa[CPW][KS];
  float w2v[CPW][16], w2s[CPW][16];
#pragma unroll
  for (int cc = 0; cc < CPW; ++cc) {
    const int c = wave + kIdxWaves * cc;
    has[cc] = c < nch;
    const int row = has[cc] ? 32 * c + ql : 0;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4 x = *reinterpret_cast<const u32x4*>(w1 + (size_t)row * X + 16 * s + 8 * half);
      if (!has[cc]) x = u32x4{0u, 0u, 0u, 0u};
      wa[cc][s] = as_bf16x8(x);
    }
    // W2 for the hidden units this lane's accumulators hold: 32 c + 8a + 4 half + b
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int h = has[cc] ? 32 * c + 8 * a + 4 * half + b : 0;
        w2v[cc][4 * a + b] = has[cc] ? __uint_as_float((uint32_t)w2[h] << 16) : 0.f;
        w2s[cc][4 * a + b] = has[cc] ? __uint_as_float((uint32_t)w2[hid + h] << 16) : 0.f;
      }
  }

  for (long long it = 0; it <= mine; ++it) {
    // this wave's loads of block `it` have landed once at most the newer
    // kIdxNst-2 blocks' are in flight; the barrier completes the block for
    // all waves and frees the stage the load below refills
    if (it < mine) __builtin_amdgcn_s_waitcnt(0x0F70 | (NDMA * (kIdxNst - 2)));
    else __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    // partial sums of the previous block -> logits
    if (it > 0 && wave == 0 && half == 0) {
      const long long row = (first + (it - 1) * stride) * kIdxRows + ql;
      const int par = (int)((it - 1) & 1);
      const float2 a0 = red[par][0][ql], a1 = red[par][1][ql], a2 = red[par][2][ql], a3 = red[par][3][ql];
      if (row < total_rows) {
        vlog[row] = (a0.x + a1.x) + (a2.x + a3.x);
        slog[row] = (a0.y + a1.y) + (a2.y + a3.y);
      }
    }
    if (it == mine) break;
    {
      const long long nb = first + (it + kIdxNst - 1) * stride;
      stage_block(nb < nblk ? nb : nblk, (int)((it + kIdxNst - 1) % kIdxNst));
#pragma unroll
      for (int i = 0; i < NDMA; ++i) asm volatile("" ::"v"(dma_off[i]));
    }
    const int st = (int)(it % kIdxNst);
    const lds_u8* xb = xbase + st * STAGEB;
    f32x16 acc[CPW];
#pragma unroll
    for (int cc = 0; cc < CPW; ++cc)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[cc][e] = 0.f;
    if (has[0]) {
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int m = s / (KS / 2), ss = s % (KS / 2);
        const bf16x8 b = *(const __attribute__((address_space(3))) bf16x8*)(xb + m * kIdxRows * ROWB + boff[ss]);
#pragma unroll
        for (int cc = 0; cc < CPW; ++cc)
          if (cc == 0 || has[cc]) acc[cc] = mfma32(wa[cc][s], b, acc[cc]);
      }
    }
    float pv = 0.f, ps = 0.f;
#pragma unroll
    for (int cc = 0; cc < CPW; ++cc)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float x = fmaxf(acc[cc][e], 0.f);
        pv = fmaf(x, w2v[cc][e], pv);
        ps = fmaf(x, w2s[cc][e], ps);
      }
    pv += swap_halves(pv);
    ps += swap_halves(ps);
    if (half == 0) red[it & 1][wave][ql] = float2{pv, ps};
  }
}

template <int D, int CPW>
void launch_index_t(dim3 grid, hipStream_t stream, const void* k, const void* v, const void* w1,
                    const void* w2, float* vlog, float* slog, long long total, int nch) {
  hipLaunchKernelGGL((index_kernel<D, CPW>), grid, dim3(kIdxThreads), 0, stream,
                     static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                     static_cast<const uint16_t*>(w1), static_cast<const uint16_t*>(w2), vlog,
                     slog, total, nch);
}

}  // namespace

hipError_t launch_index(const void* k, const void* v, int h_kv, int n, int d, int hidden,
                        const void* w1, const void* w2, float* vlog, float* slog,
                        hipStream_t stream) {
  const long long total = (long long)h_kv * n;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int c = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && c > 0)
      cus = c;
  }
  const long long blocks = (total + kIdxRows - 1) / kIdxRows;
  const dim3 grid((unsigned)(blocks < 2LL * cus ? blocks : 2LL * cus));
  const int nch = hidden / 32;
  if (d == 128) {
    if (nch <= kIdxWaves) launch_index_t<128, 1>(grid, stream, k, v, w1, w2, vlog, slog, total, nch);
    else launch_index_t<128, 2>(grid, stream, k, v, w1, w2, vlog, slog, total, nch);
  } else {
    if (nch <= kIdxWaves) launch_index_t<64, 1>(grid, stream, k, v, w1, w2, vlog, slog, total, nch);
    else launch_index_t<64, 2>(grid, stream, k, v, w1, w2, vlog, slog, total, nch);
  }
  return hipGetLastError();
}

}  // namespace vs
