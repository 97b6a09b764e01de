// mhc_coeff_bwd.hip - gfx950 kernels and the C ABI of the mHC coefficient
// backward epilogue.
//
// The operation is the epilogue of the page "perf: fuse mHC coefficient
// backward epilogue" (Liger-Kernel pull request 1402), section Summary:
// from the upstream gradients of the pre / post gates and of the
// residual-mixing logits it forms the gradient of the coefficient
// projection (grad_mix) and fixed-order sums over rows for the per-column
// bias gradients and the three gain (alpha) gradients; section Risks and
// Limitations: the sums run in a deterministic two-stage order. The page
// prints no formulas; include/mhc_coeff_bwd.h states the reading this
// library implements, bit for bit.
//
// Design for CDNA4 (MI355X):
//  * The data are small (32n + 12n^2 bytes per row: 320 at n = 4, so 2.6 MB
//    for the page's largest batch of 4 x 2048 tokens): the cost is dispatch
//    latency, not bandwidth. One wave per 64-row chunk (a lane per row,
//    every value of a row in registers) computes the chunk's sums; the
//    second stage then runs either in the same launch, by the block that
//    finishes last (an arrival counter in the workspace, release / acquire
//    fences, no waiting), or, for long batches, in a second launch with one
//    wave per summed output.
//  * The chunk sums are the first stage of the order itself (the halving
//    tree over a chunk's 64 rows, run per value by one lane after an LDS
//    transpose), and the strided walk over them plus the same tree across
//    lanes is the second, so both forms compute exactly the defined order;
//    the workspace holds the chunk sums output by output so that one
//    output's loads are contiguous across lanes.
//  * Rows past the end read as 0 through the buffer range check and produce
//    exactly +0.0 everywhere, which is what the order prescribes for them;
//    their grad_mix stores are dropped by the same check.
//  * Bit exactness: contraction off (pragma and -ffp-contract=off), no
//    fast-math, denormals kept. The post gate's sigmoid is post / c, one
//    fp32 division rounded to nearest even (hipcc's default, correctly
//    rounded division; its expansion is the only place fused multiply-adds
//    appear in this library's machine code, which the build guards check).

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <atomic>
#include <mutex>

#include "mhc_coeff_bwd.h"
#include "mhc_convert.h"
#include "mhc_lanes.h"
#include "mhc_launch.h"

#if defined(__FAST_MATH__)
#error "mhc_coeff_bwd must not be built with fast-math: its results are defined bit for bit"
#endif

#pragma clang fp contract(off)

namespace {

constexpr int kChunk = MHC_COEFF_CHUNK;  // rows per wave and per first-stage sum

__device__ __forceinline__ float ld(Rsrc rs, uint32_t byte_off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, byte_off, 0, 0));
}

__device__ __forceinline__ void st(Rsrc rs, uint32_t byte_off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rs, byte_off, 0, 0);
}

// Storage format F of the row tensors and grad_mix (MHC_COEFF_F32, _BF16,
// _F16): element bytes, the exact widening of a stored element and the
// round-to-nearest-even narrowing of a result (mhc_convert.h).
template <int F> constexpr int elem_bytes() { return F == MHC_COEFF_F32 ? 4 : 2; }

template <int F>
__device__ __forceinline__ float ld_elem(Rsrc rs, uint32_t index) {
  if constexpr (F == MHC_COEFF_F32) {
    return ld(rs, index * 4);
  } else {
    const uint16_t b = __builtin_amdgcn_raw_buffer_load_b16(rs, index * 2, 0, 0);
    return F == MHC_COEFF_BF16 ? bf16_f32(b) : f16_f32(b);
  }
}

// The fp32 value is first fixed in a register (an empty asm that takes and
// returns it): otherwise the compiler folds the product that made it into
// the fp16 conversion (v_fma_mixlo_f16), rounding once instead of rounding
// the product to fp32 and then to fp16.
template <int F>
__device__ __forceinline__ void st_elem(Rsrc rs, uint32_t index, float v) {
  if constexpr (F == MHC_COEFF_F32) {
    st(rs, index * 4, v);
  } else {
    __asm__ volatile("" : "+v"(v));
    const uint16_t b = F == MHC_COEFF_BF16 ? to_bf16(v) : to_f16(v);
    __builtin_amdgcn_raw_buffer_store_b16(b, rs, index * 2, 0, 0);
  }
}

// A lane's K consecutive stored values from element `first` (even, K even
// for 16-bit formats in the word form). WIDE (16-bit formats with every row
// tensor 4-byte aligned): two values per 32-bit access, low half first,
// which the compiler merges into wider loads and stores; otherwise one
// access per value.
template <int F, bool WIDE>
__device__ __forceinline__ float word_lo(uint32_t w) {
  return F == MHC_COEFF_BF16 ? lo_f32(w) : f16_f32(static_cast<uint16_t>(w & 0xFFFFu));
}
template <int F, bool WIDE>
__device__ __forceinline__ float word_hi(uint32_t w) {
  return F == MHC_COEFF_BF16 ? hi_f32(w) : f16_f32(static_cast<uint16_t>(w >> 16));
}

template <int F, bool WIDE, int K>
__device__ __forceinline__ void ld_row(Rsrc rs, uint32_t first, float (&out)[K]) {
  if constexpr (F == MHC_COEFF_F32 || !WIDE) {
#pragma unroll
    for (int k = 0; k < K; ++k) out[k] = ld_elem<F>(rs, first + k);
  } else {
    static_assert(K % 2 == 0, "rows hold an even number of values");
#pragma unroll
    for (int k = 0; k < K / 2; ++k) {
      const uint32_t w = __builtin_amdgcn_raw_buffer_load_b32(rs, (first + 2 * k) * 2, 0, 0);
      out[2 * k] = word_lo<F, WIDE>(w);
      out[2 * k + 1] = word_hi<F, WIDE>(w);
    }
  }
}

template <int F, bool WIDE, int K>
__device__ __forceinline__ void st_row(Rsrc rs, uint32_t first, const float (&v)[K]) {
  if constexpr (F == MHC_COEFF_F32 || !WIDE) {
#pragma unroll
    for (int k = 0; k < K; ++k) st_elem<F>(rs, first + k, v[k]);
  } else {
    // All words first, then the stores back to back (so that the compiler
    // can merge them; nothing with side effects sits between them).
    uint32_t w[K / 2];
#pragma unroll
    for (int k = 0; k < K / 2; ++k) {
      float a = v[2 * k], b = v[2 * k + 1];
      __asm__ volatile("" : "+v"(a), "+v"(b));  // as in st_elem
      w[k] = F == MHC_COEFF_BF16 ? pack_bf16x2(a, b)
                                 : static_cast<uint32_t>(to_f16(a)) |
                                       (static_cast<uint32_t>(to_f16(b)) << 16);
    }
#pragma unroll
    for (int k = 0; k < K / 2; ++k)
      __builtin_amdgcn_raw_buffer_store_b32(w[k], rs, (first + 2 * k) * 2, 0, 0);
  }
}

// The halving tree over the wave's 64 lanes: for off = 32, 16, 8, 4, 2, 1,
// x[i] += x[i + off] for i < off; lane 0 ends with the tree's sum.
template <int K>
__device__ __forceinline__ void wave_trees(float (&v)[K]) {
#pragma unroll
  for (int i = 0; i < K; ++i) v[i] = v[i] + from_lane_plus<32>(v[i]);
#pragma unroll
  for (int i = 0; i < K; ++i) v[i] = v[i] + from_lane_plus<16>(v[i]);
#pragma unroll
  for (int i = 0; i < K; ++i) v[i] = v[i] + from_lane_plus<8>(v[i]);
#pragma unroll
  for (int i = 0; i < K; ++i) v[i] = v[i] + from_lane_plus<4>(v[i]);
#pragma unroll
  for (int i = 0; i < K; ++i) v[i] = v[i] + from_lane_plus<2>(v[i]);
#pragma unroll
  for (int i = 0; i < K; ++i) v[i] = v[i] + from_lane_plus<1>(v[i]);
}

// ---------------------------------------------------------------------------
// Producer: one wave per chunk of 64 rows, lane = row.
// ---------------------------------------------------------------------------
//
// Writes grad_mix for the chunk's rows and, for each of the m + 3 summed
// quantities v (d of every column, then e of the three groups), the chunk's
// first-stage sum to partial[v * chunks + chunk].
//
// The first stage runs through LDS: every lane (row) writes its m + 3
// values into the wave's tile, value-major; then lane j reads value j's 64
// rows and applies the halving tree to them in its registers, in the order
// the tree defines (offsets 32, 16, 8, 4, 2, 1; x[i] += x[i + off] for
// i < off), and stores that chunk sum. That is the same arithmetic as a
// tree across lanes, with a third of the instructions. More than 64 values
// (n = 8) take two passes through the tile.
//
// Every wave of the block must call this (it holds block barriers); a wave
// whose chunk is past the end (`active` false) reads zeros, writes no
// grad_mix and stores no chunk sums.
constexpr int kTileStride = 68;  // floats per value row: 16-byte aligned, no bank conflicts

template <int N>
struct Tile {
  static constexpr int M = 2 * N + N * N;
  static constexpr int kValues = M + 3;
  static constexpr int kRows = kValues < 64 ? kValues : 64;  // values per pass
  static constexpr int kFloats = kRows * kTileStride;
};

template <int N, int F, bool WIDE>
__device__ __forceinline__ void chunk_sums(
    const void* __restrict__ mix, const void* __restrict__ pre, const void* __restrict__ post,
    const void* __restrict__ grad_pre, const void* __restrict__ grad_post,
    const void* __restrict__ grad_res, const float* __restrict__ alpha, float post_scale,
    void* __restrict__ grad_mix, float* __restrict__ partial, int64_t rows, uint32_t chunks,
    uint32_t c, uint32_t lane, bool active, float* tile) {
  constexpr int M = 2 * N + N * N;
  constexpr int V = M + 3;
  constexpr int64_t E = elem_bytes<F>();
  const int64_t r0 = static_cast<int64_t>(c) * kChunk;
  int64_t valid = rows - r0;
  valid = valid < 0 ? 0 : (valid > kChunk ? kChunk : valid);

  // Resources cover exactly the chunk's valid rows.
  const auto at = [r0](const void* base, int64_t width) {
    return static_cast<const char*>(base) + r0 * width * E;
  };
  const Rsrc rs_mix = make_rsrc(at(mix, M), valid * M * E);
  const Rsrc rs_pre = make_rsrc(at(pre, N), valid * N * E);
  const Rsrc rs_post = make_rsrc(at(post, N), valid * N * E);
  const Rsrc rs_gpre = make_rsrc(at(grad_pre, N), valid * N * E);
  const Rsrc rs_gpost = make_rsrc(at(grad_post, N), valid * N * E);
  const Rsrc rs_gres = make_rsrc(at(grad_res, N * N), valid * N * N * E);
  const Rsrc rs_gmix = make_rsrc(at(grad_mix, M), valid * M * E);
  const float a_pre = alpha[0], a_post = alpha[1], a_res = alpha[2];

  float d[M];
  float x[M];
  float p[N], gp[N], q[N], gq[N], gr[N * N];
  ld_row<F, WIDE>(rs_mix, lane * M, x);
  ld_row<F, WIDE>(rs_pre, lane * N, p);
  ld_row<F, WIDE>(rs_gpre, lane * N, gp);
  ld_row<F, WIDE>(rs_post, lane * N, q);
  ld_row<F, WIDE>(rs_gpost, lane * N, gq);
  ld_row<F, WIDE>(rs_gres, lane * N * N, gr);
#pragma unroll
  for (int i = 0; i < N; ++i) d[i] = gp[i] * (p[i] * (1.0f - p[i]));
#pragma unroll
  for (int i = 0; i < N; ++i) d[N + i] = gq[i] * (q[i] * (1.0f - q[i] / post_scale));
#pragma unroll
  for (int i = 0; i < N * N; ++i) d[2 * N + i] = gr[i];

  float gm[M];
#pragma unroll
  for (int j = 0; j < M; ++j) {
    const float a = j < N ? a_pre : (j < 2 * N ? a_post : a_res);
    gm[j] = a * d[j];
  }
  st_row<F, WIDE>(rs_gmix, lane * M, gm);

  float v[V];
  v[M] = 0.0f;
  v[M + 1] = 0.0f;
  v[M + 2] = 0.0f;
#pragma unroll
  for (int j = 0; j < M; ++j) {
    const int k = j < N ? 0 : (j < 2 * N ? 1 : 2);
    v[M + k] = v[M + k] + d[j] * x[j];
    v[j] = d[j];
  }

  const Rsrc rs_part = make_rsrc(partial, static_cast<int64_t>(V) * chunks * 4);
#pragma unroll
  for (int base = 0; base < V; base += 64) {
    constexpr int kRows = Tile<N>::kRows;
    const int cnt = V - base < kRows ? V - base : kRows;
    if (base > 0) __syncthreads();  // the previous pass has read the tile
#pragma unroll
    for (int i = 0; i < kRows; ++i)
      if (i < cnt) tile[i * kTileStride + lane] = v[base + i];
    __syncthreads();
    if (static_cast<int>(lane) < cnt) {
      float t[64];
      const float4* row = reinterpret_cast<const float4*>(tile + lane * kTileStride);
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const float4 f = row[q];
        t[4 * q] = f.x;
        t[4 * q + 1] = f.y;
        t[4 * q + 2] = f.z;
        t[4 * q + 3] = f.w;
      }
#pragma unroll
      for (int off = 32; off >= 1; off /= 2) {
#pragma unroll
        for (int r = 0; r < off; ++r) t[r] = t[r] + t[r + off];
      }
      if (active) st(rs_part, ((base + lane) * chunks + c) * 4, t[0]);
    }
  }
}

// Second stage for output v, by one whole wave: lane l walks the chunk sums
// l, l + 64, ... in ascending order, then the halving tree; lane 0 stores
// the result (v < m: grad_b[v], else grad_alpha[v - m]).
__device__ __forceinline__ void output_sum(const float* __restrict__ partial, uint32_t chunks,
                                           int32_t m, uint32_t v, uint32_t lane,
                                           float* __restrict__ grad_b,
                                           float* __restrict__ grad_alpha) {
  const Rsrc rs = make_rsrc(partial + static_cast<int64_t>(v) * chunks,
                            static_cast<int64_t>(chunks) * 4);
  float acc[1] = {0.0f};
  // Every lane runs the same trip count, in steps of kAhead rounds whose
  // loads are all issued before the first add (the adds stay in ascending
  // chunk order). Past the last chunk the range check reads +0.0, and
  // adding +0.0 to a sum that started at +0.0 leaves it unchanged.
  constexpr uint32_t kAhead = 8;
  const uint32_t rounds = (chunks + 63) / 64;
  for (uint32_t k = 0; k < rounds; k += kAhead) {
    float x[kAhead];
#pragma unroll
    for (uint32_t u = 0; u < kAhead; ++u) x[u] = ld(rs, ((k + u) * 64 + lane) * 4);
#pragma unroll
    for (uint32_t u = 0; u < kAhead; ++u) acc[0] = acc[0] + x[u];
  }
  wave_trees(acc);
  if (lane == 0) {
    const bool bias = static_cast<int32_t>(v) < m;
    const Rsrc out = bias ? make_rsrc(grad_b, static_cast<int64_t>(m) * 4) : make_rsrc(grad_alpha, 12);
    st(out, (bias ? v : v - m) * 4, acc[0]);
  }
}

// Two-launch form, first launch. Grid: `chunks` blocks of 64 threads.
template <int N, int F, bool WIDE>
__global__ __launch_bounds__(64) void coeff_partial_kernel(
    const void* __restrict__ mix, const void* __restrict__ pre, const void* __restrict__ post,
    const void* __restrict__ grad_pre, const void* __restrict__ grad_post,
    const void* __restrict__ grad_res, const float* __restrict__ alpha, float post_scale,
    void* __restrict__ grad_mix, float* __restrict__ partial, int64_t rows, uint32_t chunks) {
  __shared__ __align__(16) float tile[Tile<N>::kFloats];
  chunk_sums<N, F, WIDE>(mix, pre, post, grad_pre, grad_post, grad_res, alpha, post_scale,
                         grad_mix, partial, rows, chunks, blockIdx.x, threadIdx.x, true, tile);
}

// Two-launch form, second launch. Grid: m + 3 blocks of 64 threads, block v
// sums output v.
__global__ __launch_bounds__(64) void coeff_reduce_kernel(const float* __restrict__ partial,
                                                          uint32_t chunks, int32_t m,
                                                          float* __restrict__ grad_b,
                                                          float* __restrict__ grad_alpha) {
  output_sum(partial, chunks, m, blockIdx.x, threadIdx.x, grad_b, grad_alpha);
}

// One-launch form. Grid: ceil(chunks / W) blocks of 64 * W threads (W = 2
// or 4 waves); wave w of block b computes chunk b * W + w. After a barrier, one thread makes the block's chunk
// sums visible device-wide (release fence; it covers the other waves'
// stores through the barrier) and counts the block in `arrived`. The block
// that arrives last (it reads blocks - 1) fences again (acquire), computes
// every output's second stage (the outputs split over its waves) and sets
// the counter back to 0 for the next call. No block waits for another, so
// every block runs to completion whatever the others do.
template <int N, int W, int F, bool WIDE>
__global__ __launch_bounds__(64 * W) void coeff_fused_kernel(
    const void* __restrict__ mix, const void* __restrict__ pre, const void* __restrict__ post,
    const void* __restrict__ grad_pre, const void* __restrict__ grad_post,
    const void* __restrict__ grad_res, const float* __restrict__ alpha, float post_scale,
    void* __restrict__ grad_mix, float* __restrict__ partial, uint32_t* __restrict__ arrived,
    int64_t rows, uint32_t chunks, float* __restrict__ grad_b, float* __restrict__ grad_alpha) {
  constexpr int M = 2 * N + N * N;
  constexpr int Q = (M + 3 + W - 1) / W;  // outputs per wave
  __shared__ uint32_t last;
  __shared__ __align__(16) float tiles[W * Tile<N>::kFloats];
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t c = blockIdx.x * W + wave;
  chunk_sums<N, F, WIDE>(mix, pre, post, grad_pre, grad_post, grad_res, alpha, post_scale,
                         grad_mix, partial, rows, chunks, c, lane, c < chunks,
                         tiles + wave * Tile<N>::kFloats);
  __syncthreads();
  if (threadIdx.x == 0) {
    __threadfence();
    last = atomicAdd(arrived, 1u) == gridDim.x - 1;
  }
  __syncthreads();
  if (!last) return;  // the whole block
  __threadfence();
  // Outputs v = wave * Q + q. Each round loads one chunk sum per output per
  // lane (all independent), then the Q halving trees run interleaved.
  // Lanes past the last chunk add +0.0, which leaves a sum that started at
  // +0.0 unchanged; outputs past m + 3 read 0 and are not stored.
  const Rsrc rs = make_rsrc(partial, static_cast<int64_t>(M + 3) * chunks * 4);
  float acc[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) acc[q] = 0.0f;
  const uint32_t rounds = (chunks + 63) / 64;
  for (uint32_t k = 0; k < rounds; ++k) {
    const uint32_t idx = k * 64 + lane;
    const bool in = idx < chunks;
    float x[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) x[q] = ld(rs, ((wave * Q + q) * chunks + idx) * 4);
#pragma unroll
    for (int q = 0; q < Q; ++q) acc[q] = acc[q] + (in ? x[q] : 0.0f);
  }
  wave_trees(acc);
  if (lane == 0) {
    const Rsrc rb = make_rsrc(grad_b, M * 4);
    const Rsrc ra = make_rsrc(grad_alpha, 12);
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const uint32_t v = wave * Q + q;
      if (v < M) st(rb, v * 4, acc[q]);
      else if (v < M + 3) st(ra, (v - M) * 4, acc[q]);
    }
  }
  if (threadIdx.x == 0) atomicExch(arrived, 0u);
}

// One lane stores +0.0 (bit pattern 0) into the arrival counter: the set-up
// of the no-allocation entry point's scratch array on a device.
__global__ __launch_bounds__(64) void coeff_clear_counter_kernel(uint32_t* __restrict__ counter) {
  if (threadIdx.x == 0) st(make_rsrc(counter, 4), 0, 0.0f);
}

// The no-allocation entry point's workspace: a fixed array in device memory,
// one copy per GPU, held until the process ends. Host code never uses its
// name as an address (that is a host-side stand-in): the device address
// comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) uint32_t scratch[MHC_COEFF_SCRATCH_BYTES / 4];

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

thread_local char g_msg[256] = "";

mhc_status fail(mhc_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
mhc_status fail(mhc_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return s;
}

mhc_status ok() {
  g_msg[0] = '\0';
  return MHC_SUCCESS;
}

int columns(int32_t n) { return 2 * n + n * n; }

int64_t chunk_count(int64_t rows) { return (rows + kChunk - 1) / kChunk; }

// Workspace: the arrival counter of the one-launch form in the first
// kWsHeader bytes, then the chunk sums, output by output.
constexpr int64_t kWsHeader = 256;

int64_t workspace_need(int64_t rows, int32_t n) {
  if (rows == 0) return 0;
  return kWsHeader + static_cast<int64_t>(columns(n) + 3) * chunk_count(rows) * 4;
}

// The one-launch form is used at n <= 4 up to this many chunks. Measured per
// call (cold inputs, n = 4): one launch 4.6 / 5.2 / 6.9 / 8.8 us at 512 /
// 2048 / 8192 / 16384 rows against 9.0-9.2 us for two; behind from 32768
// rows (13.6 vs 9.4 us: its last block sums every output alone). At n = 8
// two launches are faster at every size measured (9.1 vs 10.5 us at 2048
// rows with 2-wave blocks, 12.2 with 4: the last block sums all 83 outputs,
// and 80-column waves sharing a CU load more slowly than one alone).
constexpr int64_t kFusedMaxChunks = 256;

struct Range {
  uintptr_t lo, hi;
  const char* name;
};

Range range(const void* p, int64_t bytes, const char* name) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + static_cast<uintptr_t>(bytes), name};
}

bool overlap(const Range& a, const Range& b) { return a.lo < b.hi && b.lo < a.hi; }

mhc_status need_ptr(const void* p, int64_t align, const char* name) {
  if (p == nullptr) return fail(MHC_ERROR_INVALID_VALUE, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(p) % align != 0)
    return fail(MHC_ERROR_INVALID_VALUE, "%s is not %lld-byte aligned", name, (long long)align);
  return ok();
}

int64_t fmt_bytes(int32_t fmt) { return fmt == MHC_COEFF_F32 ? 4 : 2; }

// Argument checks of a call. With has_workspace false (the no-allocation
// entry point), the workspace is the library's own scratch array: it is not
// checked and takes no part in the overlap tests.
mhc_status validate(const void* mix, const void* pre, const void* post, const void* grad_pre,
                    const void* grad_post, const void* grad_res, const float* alpha,
                    float post_scale, const void* grad_mix, const float* grad_b,
                    const float* grad_alpha, const void* workspace, int64_t workspace_bytes,
                    int64_t rows, int32_t n, int32_t fmt, bool has_workspace = true) {
  if (n != 2 && n != 4 && n != 8)
    return fail(MHC_ERROR_INVALID_VALUE, "the expansion rate n must be 2, 4 or 8 (got %d)", n);
  if (fmt != MHC_COEFF_F32 && fmt != MHC_COEFF_BF16 && fmt != MHC_COEFF_F16)
    return fail(MHC_ERROR_INVALID_VALUE, "dtype must be MHC_COEFF_F32, _BF16 or _F16 (got %d)",
                fmt);
  if (rows < 0 || rows > MHC_COEFF_MAX_ROWS)
    return fail(MHC_ERROR_INVALID_VALUE, "rows must be in [0, %lld] (got %lld)",
                (long long)MHC_COEFF_MAX_ROWS, (long long)rows);
  if (!(post_scale > 0.0f) || !isfinite(post_scale))
    return fail(MHC_ERROR_INVALID_VALUE, "post_scale must be finite and positive (got %g)",
                (double)post_scale);
  const int m = columns(n);
  const int64_t E = fmt_bytes(fmt);
  const int64_t need = has_workspace ? workspace_need(rows, n) : 0;
  mhc_status st;
  if ((st = need_ptr(grad_b, 4, "grad_b")) != MHC_SUCCESS) return st;
  if ((st = need_ptr(grad_alpha, 4, "grad_alpha")) != MHC_SUCCESS) return st;
  if (rows > 0) {
    const void* ps[] = {mix, pre, post, grad_pre, grad_post, grad_res, grad_mix, alpha, workspace};
    const char* names[] = {"mix", "pre", "post", "grad_pre", "grad_post", "grad_res",
                           "grad_mix", "alpha", "workspace"};
    for (int i = 0; i < (has_workspace ? 9 : 8); ++i)
      if ((st = need_ptr(ps[i], i < 7 ? E : 4, names[i])) != MHC_SUCCESS) return st;
  }
  if (workspace_bytes < need)
    return fail(MHC_ERROR_INVALID_VALUE, "workspace_bytes %lld < %lld needed",
                (long long)workspace_bytes, (long long)need);
  const Range ins[] = {range(mix, rows * m * E, "mix"), range(pre, rows * n * E, "pre"),
                       range(post, rows * n * E, "post"), range(grad_pre, rows * n * E, "grad_pre"),
                       range(grad_post, rows * n * E, "grad_post"),
                       range(grad_res, rows * n * n * E, "grad_res"),
                       range(alpha, rows > 0 ? 12 : 0, "alpha")};
  const Range outs[] = {range(grad_mix, rows * m * E, "grad_mix"), range(grad_b, m * 4, "grad_b"),
                        range(grad_alpha, 12, "grad_alpha"), range(workspace, need, "workspace")};
  const int nout = has_workspace ? 4 : 3;
  for (int a = 0; a < nout; ++a) {
    for (int b = 0; b < 7; ++b)
      if (overlap(outs[a], ins[b]))
        return fail(MHC_ERROR_ALIASING, "output %s overlaps input %s", outs[a].name, ins[b].name);
    for (int b = a + 1; b < nout; ++b)
      if (overlap(outs[a], outs[b]))
        return fail(MHC_ERROR_ALIASING, "output %s overlaps output %s", outs[a].name,
                    outs[b].name);
  }
  return ok();
}

struct CoeffArgs {
  const void *mix, *pre, *post, *grad_pre, *grad_post, *grad_res;  // stored format
  const float* alpha;
  float c;  // post_scale
  void* grad_mix;                                                   // stored format
  float *grad_b, *grad_alpha, *partial;
  uint32_t* arrived;
  int64_t rows;
  uint32_t chunks;
  int32_t fmt;
  bool wide;  // 16-bit formats: every row tensor 4-byte aligned (32-bit accesses)
};

template <int N, int F, bool WIDE>
hipError_t launch_partial_f(const CoeffArgs& a, hipStream_t s, hipEvent_t start) {
  return launch_kernel(coeff_partial_kernel<N, F, WIDE>, dim3(a.chunks), dim3(64), s, start,
                       nullptr, a.mix, a.pre, a.post, a.grad_pre, a.grad_post, a.grad_res,
                       a.alpha, a.c, a.grad_mix, a.partial, a.rows, a.chunks);
}

template <int N>
hipError_t launch_partial(const CoeffArgs& a, hipStream_t s, hipEvent_t start) {
  switch (a.fmt) {
    case MHC_COEFF_BF16:
      return a.wide ? launch_partial_f<N, MHC_COEFF_BF16, true>(a, s, start)
                    : launch_partial_f<N, MHC_COEFF_BF16, false>(a, s, start);
    case MHC_COEFF_F16:
      return a.wide ? launch_partial_f<N, MHC_COEFF_F16, true>(a, s, start)
                    : launch_partial_f<N, MHC_COEFF_F16, false>(a, s, start);
    default: return launch_partial_f<N, MHC_COEFF_F32, false>(a, s, start);
  }
}

// Waves per block of the one-launch form: 2 up to this many chunks, 4
// above. Measured per call (cold inputs, n = 4): 2-wave blocks 4.5 / 4.9 /
// 5.1 / 5.5 / 5.6 us at 512 / 1024 / 2048 / 3072 / 4096 rows against 5.0 /
// 5.2 / 5.6 / 5.7 / 5.7 us with 4 (more CUs share the first stage); 4-wave
// blocks 7.1 / 8.8 us at 8192 / 16384 rows against 7.3 / 10.0 us (the last
// block's waves each sum fewer outputs). At n = 2 the same or better.
constexpr uint32_t kTwoWaveMaxChunks = 64;

template <int N, int W, int F, bool WIDE>
hipError_t launch_fused_w(const CoeffArgs& a, hipStream_t s, hipEvent_t start, hipEvent_t stop) {
  const uint32_t blocks = (a.chunks + W - 1) / W;
  return launch_kernel(coeff_fused_kernel<N, W, F, WIDE>, dim3(blocks), dim3(64 * W), s, start,
                       stop, a.mix, a.pre, a.post, a.grad_pre, a.grad_post, a.grad_res, a.alpha,
                       a.c, a.grad_mix, a.partial, a.arrived, a.rows, a.chunks, a.grad_b,
                       a.grad_alpha);
}

template <int N, int F, bool WIDE>
hipError_t launch_fused_f(const CoeffArgs& a, hipStream_t s, hipEvent_t start, hipEvent_t stop) {
  if (a.chunks <= kTwoWaveMaxChunks) return launch_fused_w<N, 2, F, WIDE>(a, s, start, stop);
  return launch_fused_w<N, 4, F, WIDE>(a, s, start, stop);
}

template <int N>
hipError_t launch_fused(const CoeffArgs& a, hipStream_t s, hipEvent_t start, hipEvent_t stop) {
  switch (a.fmt) {
    case MHC_COEFF_BF16:
      return a.wide ? launch_fused_f<N, MHC_COEFF_BF16, true>(a, s, start, stop)
                    : launch_fused_f<N, MHC_COEFF_BF16, false>(a, s, start, stop);
    case MHC_COEFF_F16:
      return a.wide ? launch_fused_f<N, MHC_COEFF_F16, true>(a, s, start, stop)
                    : launch_fused_f<N, MHC_COEFF_F16, false>(a, s, start, stop);
    default: return launch_fused_f<N, MHC_COEFF_F32, false>(a, s, start, stop);
  }
}

// Launches of one call: 1 = one launch (chunk sums + last-block reduction),
// 2 = chunk-sum launch then reduction launch. 0 lets the policy choose.
int plan_launches(int64_t rows, int32_t n, int32_t launches) {
  if (rows == 0) return 2;  // only the reduction launch runs: it writes the +0.0 sums
  if (launches != 0) return launches;
  return n <= 4 && chunk_count(rows) <= kFusedMaxChunks ? 1 : 2;
}

// The status of one launch (the value hipExtLaunchKernel returned for it).
mhc_status launch_status(hipError_t e, const char* what) {
  if (e != hipSuccess)
    return fail(MHC_ERROR_HIP, "%s launch failed: %s (%s)", what, hipGetErrorName(e),
                hipGetErrorString(e));
  return ok();
}

// The arguments of a call whose pointers and sizes have been validated;
// `workspace` is device memory of at least workspace_need(rows, n) bytes
// whose first 4 bytes (the arrival counter) are zero.
CoeffArgs make_args(const void* mix, const void* pre, const void* post, const void* grad_pre,
                    const void* grad_post, const void* grad_res, const float* alpha,
                    float post_scale, void* grad_mix, float* grad_b, float* grad_alpha,
                    void* workspace, int64_t rows, int32_t fmt) {
  CoeffArgs a;
  a.mix = mix; a.pre = pre; a.post = post; a.grad_pre = grad_pre; a.grad_post = grad_post;
  a.grad_res = grad_res; a.alpha = alpha;
  a.c = post_scale;
  a.grad_mix = grad_mix; a.grad_b = grad_b; a.grad_alpha = grad_alpha;
  a.arrived = static_cast<uint32_t*>(workspace);
  a.partial = rows > 0 ? reinterpret_cast<float*>(static_cast<char*>(workspace) + kWsHeader)
                       : nullptr;
  a.rows = rows;
  a.chunks = static_cast<uint32_t>(chunk_count(rows));
  a.fmt = fmt;
  // Rows hold an even number of values at every n (2n + n^2, n and n^2),
  // so with 4-byte-aligned bases every row starts 4-byte aligned.
  a.wide = true;
  for (const void* t : {mix, pre, post, grad_pre, grad_post, grad_res,
                        static_cast<const void*>(grad_mix)})
    if (reinterpret_cast<uintptr_t>(t) % 4 != 0) a.wide = false;
  return a;
}

// Enqueue one call's kernels (one launch or two, as planned).
mhc_status run(const CoeffArgs& a, int32_t n, int32_t launches, hipStream_t s, hipEvent_t start,
               hipEvent_t stop) {
  mhc_status st;
  if (plan_launches(a.rows, n, launches) == 1) {
    hipError_t e;
    switch (n) {
      case 2: e = launch_fused<2>(a, s, start, stop); break;
      case 4: e = launch_fused<4>(a, s, start, stop); break;
      default: e = launch_fused<8>(a, s, start, stop); break;
    }
    return launch_status(e, "coefficient backward (one launch)");
  }
  if (a.chunks > 0) {
    hipError_t e;
    switch (n) {
      case 2: e = launch_partial<2>(a, s, start); break;
      case 4: e = launch_partial<4>(a, s, start); break;
      default: e = launch_partial<8>(a, s, start); break;
    }
    if ((st = launch_status(e, "coefficient backward (chunk sums)")) != MHC_SUCCESS) return st;
  }
  const int32_t m = columns(n);
  const hipError_t e =
      launch_kernel(coeff_reduce_kernel, dim3(m + 3), dim3(64), s, a.chunks > 0 ? nullptr : start,
                    stop, a.partial, a.chunks, m, a.grad_b, a.grad_alpha);
  return launch_status(e, "coefficient backward (reduction)");
}

// The scratch array's device address on each device, looked up once per
// device with that device current, and whether its arrival counter has been
// cleared there.
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
std::atomic<bool> g_scratch_cleared[kMaxDevices];

// The current device's scratch address; on the first call on a device, also
// enqueue on `s` the kernel that zeroes its arrival counter (device memory
// starts zeroed at load; clearing once more makes the first call independent
// of that).
mhc_status device_scratch(hipStream_t s, void** out) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return fail(MHC_ERROR_HIP, "hipGetDevice failed: %s", hipGetErrorName(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MHC_ERROR_INVALID_VALUE, "device %d is beyond the %d devices supported", dev,
                kMaxDevices);
  std::call_once(g_scratch_once[dev], [dev] {
    void* ptr = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = ptr;
  });
  if (g_scratch_err[dev] != hipSuccess || g_scratch_ptr[dev] == nullptr)
    return fail(MHC_ERROR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                hipGetErrorName(g_scratch_err[dev]));
  if (!g_scratch_cleared[dev].exchange(true)) {
    const hipError_t c = launch_kernel(coeff_clear_counter_kernel, dim3(1), dim3(64), s, nullptr,
                                       nullptr, static_cast<uint32_t*>(g_scratch_ptr[dev]));
    if (c != hipSuccess) {
      g_scratch_cleared[dev] = false;
      return launch_status(c, "coefficient backward (scratch set-up)");
    }
  }
  *out = g_scratch_ptr[dev];
  return ok();
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------

extern "C" {

int mhc_coeff_abi_version(void) { return MHC_COEFF_ABI_VERSION; }

const char* mhc_coeff_last_error_message(void) { return g_msg; }

int64_t mhc_coeff_bwd_workspace_bytes(int64_t rows, int32_t n) {
  if ((n != 2 && n != 4 && n != 8) || rows < 0 || rows > MHC_COEFF_MAX_ROWS) return -1;
  return workspace_need(rows, n);
}

mhc_status mhc_coeff_bwd_validate(const float* mix, const float* pre, const float* post,
                                  const float* grad_pre, const float* grad_post,
                                  const float* grad_res, const float* alpha, float post_scale,
                                  const float* grad_mix, const float* grad_b,
                                  const float* grad_alpha, const void* workspace,
                                  int64_t workspace_bytes, int64_t rows, int32_t n) {
  return validate(mix, pre, post, grad_pre, grad_post, grad_res, alpha, post_scale, grad_mix,
                  grad_b, grad_alpha, workspace, workspace_bytes, rows, n, MHC_COEFF_F32);
}

mhc_status mhc_coeff_bwd_validate_ex(const void* mix, const void* pre, const void* post,
                                     const void* grad_pre, const void* grad_post,
                                     const void* grad_res, const float* alpha, float post_scale,
                                     const void* grad_mix, const float* grad_b,
                                     const float* grad_alpha, const void* workspace,
                                     int64_t workspace_bytes, int64_t rows, int32_t n,
                                     int32_t dtype) {
  return validate(mix, pre, post, grad_pre, grad_post, grad_res, alpha, post_scale, grad_mix,
                  grad_b, grad_alpha, workspace, workspace_bytes, rows, n, dtype);
}

int32_t mhc_coeff_bwd_plan(int64_t rows, int32_t n, int32_t launches) {
  if ((n != 2 && n != 4 && n != 8) || rows < 0 || rows > MHC_COEFF_MAX_ROWS ||
      launches < 0 || launches > 2)
    return -1;
  return plan_launches(rows, n, launches);
}

mhc_status mhc_coeff_bwd_ex(const void* mix, const void* pre, const void* post,
                            const void* grad_pre, const void* grad_post, const void* grad_res,
                            const float* alpha, float post_scale, void* grad_mix, float* grad_b,
                            float* grad_alpha, void* workspace, int64_t workspace_bytes,
                            int64_t rows, int32_t n, int32_t dtype, int32_t launches,
                            void* stream, void* start_event, void* stop_event) {
  mhc_status st = validate(mix, pre, post, grad_pre, grad_post, grad_res, alpha, post_scale,
                           grad_mix, grad_b, grad_alpha, workspace, workspace_bytes, rows, n,
                           dtype);
  if (st != MHC_SUCCESS) return st;
  if (launches < 0 || launches > 2)
    return fail(MHC_ERROR_INVALID_VALUE, "launches must be 0, 1 or 2 (got %d)", launches);
  const CoeffArgs a = make_args(mix, pre, post, grad_pre, grad_post, grad_res, alpha, post_scale,
                                grad_mix, grad_b, grad_alpha, workspace, rows, dtype);
  return run(a, n, launches, static_cast<hipStream_t>(stream),
             static_cast<hipEvent_t>(start_event), static_cast<hipEvent_t>(stop_event));
}

mhc_status mhc_coeff_bwd(const float* mix, const float* pre, const float* post,
                         const float* grad_pre, const float* grad_post, const float* grad_res,
                         const float* alpha, float post_scale, float* grad_mix, float* grad_b,
                         float* grad_alpha, void* workspace, int64_t workspace_bytes,
                         int64_t rows, int32_t n, int32_t launches, void* stream,
                         void* start_event, void* stop_event) {
  return mhc_coeff_bwd_ex(mix, pre, post, grad_pre, grad_post, grad_res, alpha, post_scale,
                          grad_mix, grad_b, grad_alpha, workspace, workspace_bytes, rows, n,
                          MHC_COEFF_F32, launches, stream, start_event, stop_event);
}

mhc_status mhc_coeff_bwd_noalloc(const float* mix, const float* pre, const float* post,
                                 const float* grad_pre, const float* grad_post,
                                 const float* grad_res, const float* alpha, float post_scale,
                                 float* grad_mix, float* grad_b, float* grad_alpha, int64_t rows,
                                 int32_t n, int32_t launches, void* stream, void* start_event,
                                 void* stop_event) {
  // Sizes first, on the host alone: nothing is touched for a call that
  // does not fit the scratch array.
  if (n != 2 && n != 4 && n != 8)
    return fail(MHC_ERROR_INVALID_VALUE, "the expansion rate n must be 2, 4 or 8 (got %d)", n);
  if (rows < 0 || rows > MHC_COEFF_MAX_ROWS)
    return fail(MHC_ERROR_INVALID_VALUE, "rows must be in [0, %lld] (got %lld)",
                (long long)MHC_COEFF_MAX_ROWS, (long long)rows);
  const int64_t need = workspace_need(rows, n);
  if (need > MHC_COEFF_SCRATCH_BYTES)
    return fail(MHC_ERROR_INVALID_VALUE,
                "%lld rows at n=%d need %lld bytes of workspace, more than the %lld-byte scratch "
                "array of the no-allocation entry point (use mhc_coeff_bwd with a workspace)",
                (long long)rows, n, (long long)need, (long long)MHC_COEFF_SCRATCH_BYTES);
  if (launches < 0 || launches > 2)
    return fail(MHC_ERROR_INVALID_VALUE, "launches must be 0, 1 or 2 (got %d)", launches);
  // Every other argument as mhc_coeff_bwd checks it.
  mhc_status st = validate(mix, pre, post, grad_pre, grad_post, grad_res, alpha, post_scale,
                           grad_mix, grad_b, grad_alpha, nullptr, 0, rows, n, MHC_COEFF_F32,
                           false);
  if (st != MHC_SUCCESS) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if (rows > 0 && (st = device_scratch(s, &ws)) != MHC_SUCCESS) return st;
  const CoeffArgs a = make_args(mix, pre, post, grad_pre, grad_post, grad_res, alpha, post_scale,
                                grad_mix, grad_b, grad_alpha, ws, rows, MHC_COEFF_F32);
  return run(a, n, launches, s, static_cast<hipEvent_t>(start_event),
             static_cast<hipEvent_t>(stop_event));
}

}  // extern "C"
