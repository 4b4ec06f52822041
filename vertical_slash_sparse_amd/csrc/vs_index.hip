// vs_index.hip -- VSIndexer scoring for gfx950.
//
// VSPrefill (gist.science summaries of arXiv 2603.04460, English page,
// Technical Summary section 2, "Key Components 1. VSIndexer"): a
// shared-weight two-layer linear network over concat(K with RoPE, V) with
// separate down-projection heads for vertical and slash importance:
//     h_j = max(0, W1 [k_j | v_j]),   vlog_j = W2[0] . h_j,   slog_j = W2[1] . h_j.
//
// Each position reads 2*d*2 = 512 bytes and costs 2*256*128 + 2*2*128 flops,
// about 128 flop per byte -- under the MI355X ridge (~315 flop/B for bf16
// MFMA against 8 TB/s), so the kernel is HBM-bound and is built to stream:
//  * a workgroup of four waves takes 32 consecutive positions at a time; their
//    K and V rows (16 KiB, contiguous in HBM) arrive by LDS-DMA into a ring of
//    four stages, so every HBM read is a full 1 KiB line run and three blocks
//    are in flight while one is multiplied;
//  * wave w owns hidden units 32w .. 32w+31: its slice of W1 (the A operand of
//    H^T = W1 X^T on v_mfma_f32_32x32x16_bf16) and of W2 stay in registers for
//    the whole kernel, and the 32 positions are the B operand, read from LDS;
//  * the second layer runs in fp32 on the vector ALUs from the fp32
//    accumulators; the four waves' partial sums meet in LDS and are added
//    after the next block's barrier, so each block costs one barrier.
#include "vs_common.h"
#include "vs_internal.h"

namespace vs {

namespace {

constexpr int kIdxD = 128;            // head dim
constexpr int kIdxX = 2 * kIdxD;      // indexer input width
constexpr int kIdxH = 128;            // hidden width
constexpr int kIdxKS = kIdxX / 16;    // k-steps of the first layer
constexpr int kIdxRows = 32;          // positions per block
constexpr int kIdxRowB = kIdxD * 2;   // bytes of one K (or V) row
constexpr int kIdxStageB = 2 * kIdxRows * kIdxRowB;  // K rows then V rows
constexpr int kIdxNst = 4;            // ring stages
constexpr int kIdxThreads = 256;
constexpr int kIdxDma = kIdxStageB / 1024 / (kIdxThreads / 64);  // 1 KiB loads per wave per block

// XOR swizzle of the 16-byte chunks of a 256-byte row, so that 32 lanes
// reading one chunk of 32 consecutive rows hit distinct banks
__device__ __forceinline__ int idx_swz(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }

__global__ __launch_bounds__(kIdxThreads, 2) void index_kernel(const uint16_t* __restrict__ k,
                                                               const uint16_t* __restrict__ v,
                                                               const uint16_t* __restrict__ w1,
                                                               const uint16_t* __restrict__ w2,
                                                               float* __restrict__ vlog,
                                                               float* __restrict__ slog,
                                                               long long total_rows) {
  __shared__ __align__(16) uint8_t xs[kIdxNst * kIdxStageB];
  __shared__ float2 red[2][4][kIdxRows];  // [block parity][wave][position] partial (vertical, slash)
  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  lds_u8* const xbase = (lds_u8*)xs;

  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, ql = lane & 31;
  const int wave = wave_uniform(tid >> 6);

  // DMA: wave w moves kIdxDma KiB of each block; a KiB holds 4 rows, lane l
  // row (l / 16) of them, chunk slot l % 16, which holds source chunk
  // slot ^ swizzle(row)
  const uint32_t rbytes = (uint32_t)(total_rows * kIdxRowB);
  const u32x4 wk = buffer_words(k, rbytes);
  const u32x4 wv = buffer_words(v, rbytes);
  int dma_lds[kIdxDma], dma_src[kIdxDma], dma_mat[kIdxDma];
#pragma unroll
  for (int i = 0; i < kIdxDma; ++i) {
    const int kib = wave * kIdxDma + i;   // 0..15: K rows 0..31 in KiB 0..7, V rows in 8..15
    const int mat = kib >= 8 ? 1 : 0;
    const int r = 4 * (kib & 7) + lane / 16;
    dma_mat[i] = mat;
    dma_lds[i] = kib * 1024;
    dma_src[i] = r * kIdxRowB + 16 * ((lane & 15) ^ idx_swz(r));
  }
  unsigned dma_off[kIdxDma];
  auto stage_block = [&](long long blk, int st) {
    const unsigned base = (unsigned)(blk * kIdxRows * kIdxRowB);  // past the end: out of range, zeros
#pragma unroll
    for (int i = 0; i < kIdxDma; ++i) {
      const unsigned off = blk * kIdxRows < total_rows ? base + (unsigned)dma_src[i] : rbytes;
      dma16(dma_mat[i] ? wv : wk, (uint32_t)(uintptr_t)(xbase + st * kIdxStageB + dma_lds[i]), off);
      dma_off[i] = off;
    }
  };
  // B operand (k-step s) of block stage st: position ql, chunk 2s' + half
  int boff[kIdxKS / 2];
#pragma unroll
  for (int s = 0; s < kIdxKS / 2; ++s) boff[s] = ql * kIdxRowB + 16 * ((2 * s + half) ^ idx_swz(ql));

  const long long nblk = (total_rows + kIdxRows - 1) / kIdxRows;
  const long long first = blockIdx.x, stride = gridDim.x;
  if (first >= nblk) return;
  const long long mine = (nblk - first + stride - 1) / stride;  // blocks of this workgroup
  for (int j = 0; j < kIdxNst - 1; ++j) stage_block(first + j * stride < nblk ? first + j * stride : nblk, j);

  // The first blocks' loads are already in flight: the weights' own latency
  // (they come from L2 or HBM on a call's first use) overlaps them.
  // W1 rows 32*wave + ql as A operands (k-step s: input dims 16s + 8*half ..)
  bf16x8 wa[kIdxKS];
#pragma unroll
  for (int s = 0; s < kIdxKS; ++s)
    wa[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(w1 + (size_t)(32 * wave + ql) * kIdxX + 16 * s + 8 * half));
  // W2 for the hidden units this lane's accumulators hold: 32*wave + 8a + 4*half + b
  float w2v[16], w2s[16];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int h = 32 * wave + 8 * a + 4 * half + b;
      w2v[4 * a + b] = __uint_as_float((uint32_t)w2[h] << 16);
      w2s[4 * a + b] = __uint_as_float((uint32_t)w2[kIdxH + h] << 16);
    }

  for (long long it = 0; it <= mine; ++it) {
    // this wave's loads of block `it` have landed once at most the newer
    // kIdxNst-2 blocks' are in flight; the barrier completes the block for
    // all waves and frees the stage the load below refills
    if (it < mine) __builtin_amdgcn_s_waitcnt(0x0F70 | (kIdxDma * (kIdxNst - 2)));
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
      for (int i = 0; i < kIdxDma; ++i) asm volatile("" ::"v"(dma_off[i]));
    }
    const int st = (int)(it % kIdxNst);
    const lds_u8* xb = xbase + st * kIdxStageB;
    f32x16 acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
    for (int s = 0; s < kIdxKS; ++s) {
      const int m = s / (kIdxKS / 2), ss = s % (kIdxKS / 2);
      const bf16x8 b = *(const __attribute__((address_space(3))) bf16x8*)(xb + m * kIdxRows * kIdxRowB + boff[ss]);
      acc = mfma32(wa[s], b, acc);
    }
    float pv = 0.f, ps = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float x = fmaxf(acc[e], 0.f);
      pv = fmaf(x, w2v[e], pv);
      ps = fmaf(x, w2s[e], ps);
    }
    pv += swap_halves(pv);
    ps += swap_halves(ps);
    if (half == 0) red[it & 1][wave][ql] = float2{pv, ps};
  }
}

}  // namespace

hipError_t launch_index(const void* k, const void* v, int h_kv, int n, const void* w1,
                        const void* w2, float* vlog, float* slog, hipStream_t stream) {
  const long long total = (long long)h_kv * n;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int c = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && c > 0)
      cus = c;
  }
  const long long blocks = (total + kIdxRows - 1) / kIdxRows;
  const long long grid = blocks < 2LL * cus ? blocks : 2LL * cus;
  hipLaunchKernelGGL(index_kernel, dim3((unsigned)grid), dim3(kIdxThreads), 0, stream,
                     static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                     static_cast<const uint16_t*>(w1), static_cast<const uint16_t*>(w2), vlog,
                     slog, total);
  return hipGetLastError();
}

}  // namespace vs
