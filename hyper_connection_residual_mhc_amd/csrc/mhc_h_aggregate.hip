// mhc_h_aggregate.hip - gfx950 kernels and the C ABI of the mHC pre /
// H-aggregate operation (forward) and its backward.
//
// The operation and its arithmetic contract are those of the page "Add
// batch-invariant h_aggregate kernel" (RL-Kernel pull request 366),
// sections Summary and Batch invariance; the backward is the derivative of
// that formula, which the page's review comments ask for. The public header
// include/mhc_h_aggregate.h states both in full.
//
// Design for CDNA4 (MI355X):
//  * The path is a stream over HBM (about 0.7 flop per byte), so it is laid
//    out for coalesced 16-byte vector accesses per lane, many bytes in flight
//    per CU and no reuse to cache. MFMA has no role: nothing is a
//    contraction.
//  * Forward: a block covers a contiguous slice of one token's hidden axis,
//    so the token index, pre[t,:] and every base address are wave-uniform
//    (scalar registers and scalar loads). Each lane owns one or more
//    V-element units and is their only writer; no lane ever reduces.
//  * Backward, two layouts of the same fixed summation order: for long
//    batches one wave streams one (token, stream) row, each lane holding
//    four of the order's 256 accumulator lanes, and reduces it in registers;
//    for short batches the 256 accumulator lanes are a block's 256 threads
//    and the last stage goes through LDS. Both write grad_residual on the
//    way.
//  * Bit exactness: contraction is off for the whole file (pragma and
//    -ffp-contract=off), fast-math builds are refused, fp32 denormals are
//    kept (the kernel descriptor's default mode), and every bf16 result goes
//    through the hardware round-to-nearest-even pack conversion.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <atomic>

#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "mhc_convert.h"
#include "mhc_h_aggregate.h"
#include "mhc_lanes.h"
#include "mhc_launch.h"

#if defined(__FAST_MATH__)
#error "mhc_h_aggregate must not be built with fast-math: its results are defined bit for bit"
#endif

#pragma clang fp contract(off)

namespace {

// ---------------------------------------------------------------------------
// Device helpers: V-element vectors (conversions in mhc_convert.h)
// ---------------------------------------------------------------------------

// A V-element bf16 vector as a native vector of 32-bit words (V = 8, 4), one
// word (V = 2) or one half-word (V = 1).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
template <int V> struct Vec;
template <> struct Vec<8> { typedef u32x4 type; };
template <> struct Vec<4> { typedef u32x2 type; };
template <> struct Vec<2> { typedef uint32_t type; };
template <> struct Vec<1> { typedef uint16_t type; };

// Element e (compile-time after unrolling) of a vector, widened to fp32.
template <int V>
__device__ __forceinline__ float elem(const typename Vec<V>::type& v, int e);
template <> __device__ __forceinline__ float elem<8>(const u32x4& v, int e) {
  const uint32_t w = v[e >> 1];
  return (e & 1) ? hi_f32(w) : lo_f32(w);
}
template <> __device__ __forceinline__ float elem<4>(const u32x2& v, int e) {
  const uint32_t w = v[e >> 1];
  return (e & 1) ? hi_f32(w) : lo_f32(w);
}
template <> __device__ __forceinline__ float elem<2>(const uint32_t& v, int e) {
  return (e & 1) ? hi_f32(v) : lo_f32(v);
}
template <> __device__ __forceinline__ float elem<1>(const uint16_t& v, int) {
  return bf16_f32(v);
}

// V fp32 values -> one bf16 vector.
template <int V>
__device__ __forceinline__ typename Vec<V>::type pack(const float (&y)[V]);
template <> __device__ __forceinline__ u32x4 pack<8>(const float (&y)[8]) {
  return u32x4{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]),
               pack_bf16x2(y[6], y[7])};
}
template <> __device__ __forceinline__ u32x2 pack<4>(const float (&y)[4]) {
  return u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
}
template <> __device__ __forceinline__ uint32_t pack<2>(const float (&y)[2]) {
  return pack_bf16x2(y[0], y[1]);
}
template <> __device__ __forceinline__ uint16_t pack<1>(const float (&y)[1]) {
  return to_bf16(y[0]);
}

// Memory access: CDNA buffer instructions. A row (or a token's rows) is
// described by a buffer resource (make_rsrc in mhc_lanes.h: base address and
// byte length, held in scalar registers, wave-uniform), each lane supplies
// one 32-bit byte offset.
// Accesses past the resource's length are dropped by the hardware (loads
// return 0), so no lane can touch memory outside the row it was given.
// Streamed bytes are touched once, so loads carry the nontemporal hint; the
// one row several waves read (the backward's grad_out in the row layout)
// keeps the default policy so that it stays in cache for them.
// (kNontemporal, kCached and kWriteThrough in mhc_lanes.h.) Stores: the
// forward's output is written through at device scope (sc1); measured with
// cold caches, the forward (4 bytes read per byte written) streams 5-8%
// faster with it than with nt; the backward (5:4) and the accumulating
// backward (9:4) stream 2-4% slower, so they keep nt.

// Load V bf16 elements at element `off` (per lane) plus `soff` bytes
// (wave-uniform, carried in a scalar register) from the resource, with
// cache-policy bits POL.
template <int V, int POL = kNontemporal>
__device__ __forceinline__ typename Vec<V>::type load_vec(Rsrc rs, uint32_t off, uint32_t soff) {
  if constexpr (V == 8) {
    return __builtin_amdgcn_raw_buffer_load_b128(rs, off * 2, soff, POL);
  } else if constexpr (V == 4) {
    return __builtin_amdgcn_raw_buffer_load_b64(rs, off * 2, soff, POL);
  } else if constexpr (V == 2) {
    return __builtin_amdgcn_raw_buffer_load_b32(rs, off * 2, soff, POL);
  } else {
    static_assert(V == 1, "vector width");
    return __builtin_amdgcn_raw_buffer_load_b16(rs, off * 2, soff, POL);
  }
}

// Stores take no scalar offset: the whole byte offset travels in the VGPR.
// A store of more than 8 bytes reads its data registers over several cycles,
// and an instruction right after it must not overwrite them. The compiler
// inserts that wait state for stores whose scalar offset is the constant 0,
// but not for stores with a scalar-register offset, and gfx950 needs it in
// both cases (a register-offset dwordx4 store followed at once by a write to
// its second data register was measured to store the new value from the
// last lanes of each 16). tests/test_build_guards.py checks the machine code
// for this pattern.
// POL: cache-policy bits of the store (kNontemporal or kWriteThrough).
template <int V, int POL>
__device__ __forceinline__ void store_vec(Rsrc rs, uint32_t off, const typename Vec<V>::type& v) {
  if constexpr (V == 8) {
    __builtin_amdgcn_raw_buffer_store_b128(v, rs, off * 2, 0, POL);
  } else if constexpr (V == 4) {
    __builtin_amdgcn_raw_buffer_store_b64(v, rs, off * 2, 0, POL);
  } else if constexpr (V == 2) {
    __builtin_amdgcn_raw_buffer_store_b32(v, rs, off * 2, 0, POL);
  } else {
    static_assert(V == 1, "vector width");
    __builtin_amdgcn_raw_buffer_store_b16(v, rs, off * 2, 0, POL);
  }
}

// ---------------------------------------------------------------------------
// Forward kernel
// ---------------------------------------------------------------------------
//
// Grid: (blocks_per_token, T) blocks of blockDim.x threads (a multiple of
// 64). Block (c, t) serves token t and, within it, the units
// [c * blockDim.x * UPT, (c + 1) * blockDim.x * UPT); a unit is V consecutive
// hidden elements. Lane x of the block owns units
// c*blockDim.x*UPT + k*blockDim.x + x for k < UPT, so every load and store
// instruction of a wave covers 64 consecutive units. All loads of a lane are
// issued before any arithmetic.
//
// N is the expansion rate (residual streams): 4 on the page, 2 and 8 for the
// generalised operation. The N products are summed as a balanced pairwise
// tree: adjacent pairs first, then pairs of pairs - (0+1)+(2+3) for N = 4.
template <int V, int UPT, int N>
__global__ __launch_bounds__(1024) void hagg_fwd_kernel(
    const uint16_t* __restrict__ residual, const float* __restrict__ pre,
    uint16_t* __restrict__ out, int64_t H, uint32_t block_threads) {
  typedef typename Vec<V>::type VT;
  const uint32_t c = blockIdx.x;
  const uint32_t t = blockIdx.y;

  const float* p = pre + N * static_cast<int64_t>(t);
  float w[N];
#pragma unroll
  for (int i = 0; i < N; ++i) w[i] = p[i];
  // One resource per row: the token's N residual rows and its output row
  // (2H bytes each). Units past the end of the row read zeros and their
  // stores are dropped by the range check, so no lane branches: every
  // argument is fetched at once and the loads issue right after.
  Rsrc res[N];
#pragma unroll
  for (int i = 0; i < N; ++i) res[i] = make_rsrc(residual + (static_cast<int64_t>(t) * N + i) * H, 2 * H);
  const Rsrc o = make_rsrc(out + static_cast<int64_t>(t) * H, 2 * H);

  const uint32_t first = c * block_threads * UPT + threadIdx.x;

  VT x[N][UPT];
#pragma unroll
  for (int k = 0; k < UPT; ++k) {
    const uint32_t h = (first + k * block_threads) * V;
#pragma unroll
    for (int i = 0; i < N; ++i) x[i][k] = load_vec<V>(res[i], h, 0);
  }
#pragma unroll
  for (int k = 0; k < UPT; ++k) {
    const uint32_t h = (first + k * block_threads) * V;
    float y[V];
#pragma unroll
    for (int e = 0; e < V; ++e) {
      // Separate fp32 round-to-nearest products, then the pairwise tree
      // of separate round-to-nearest sums.
      float lv[N];
#pragma unroll
      for (int i = 0; i < N; ++i) lv[i] = w[i] * elem<V>(x[i][k], e);
#pragma unroll
      for (int width = N; width > 1; width /= 2) {
#pragma unroll
        for (int j = 0; j < width / 2; ++j) lv[j] = lv[2 * j] + lv[2 * j + 1];
      }
      y[e] = lv[0];
    }
    store_vec<V, kWriteThrough>(o, h, pack<V>(y));
  }
}

// ---------------------------------------------------------------------------
// Backward kernel
// ---------------------------------------------------------------------------

constexpr int kGroup = 8;
constexpr int kLanes = 256;

// The register slots of the backward's ring of loads: for each of U groups,
// the grad_out vector(s), the S residual vectors and (accumulating form) the
// S stored-gradient vectors of its 8 elements.
template <int V, int U, int S, bool ACC>
struct BwdSlots {
  typedef typename Vec<V>::type VT;
  static constexpr int NV = kGroup / V;  // accesses per group
  VT g[U][NV];
  VT r[U][NV][S];
  VT old[ACC ? U : 1][NV][S];
};

// Issue the loads of group k into slot u (u is a constant after unrolling).
template <int V, int U, int S, bool ACC>
__device__ __forceinline__ void bwd_issue(BwdSlots<V, U, S, ACC>& sl, int u, uint32_t k,
                                          Rsrc g_row, const Rsrc (&r_row)[S],
                                          const Rsrc (&gr_row)[S]) {
#pragma unroll
  for (int v = 0; v < BwdSlots<V, U, S, ACC>::NV; ++v) {
    const uint32_t h = k * kGroup + v * V;
    sl.g[u][v] = load_vec<V>(g_row, h, 0);
#pragma unroll
    for (int i = 0; i < S; ++i) sl.r[u][v][i] = load_vec<V>(r_row[i], h, 0);
    if constexpr (ACC) {
#pragma unroll
      for (int i = 0; i < S; ++i) sl.old[u][v][i] = load_vec<V>(gr_row[i], h, 0);
    }
  }
}

// Consume slot u holding group k: write its grad_residual vectors and add
// its products to the accumulators, element by element in ascending h.
// Stream by stream, so only one stream's results are live at a time.
template <int V, int U, int S, bool ACC>
__device__ __forceinline__ void bwd_consume(BwdSlots<V, U, S, ACC>& sl, int u, uint32_t k,
                                            const float (&w)[S], float (&acc)[S],
                                            const Rsrc (&gr_row)[S]) {
#pragma unroll
  for (int v = 0; v < BwdSlots<V, U, S, ACC>::NV; ++v) {
    const uint32_t h = k * kGroup + v * V;
#pragma unroll
    for (int i = 0; i < S; ++i) {
      float gr[V];
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const float ge = elem<V>(sl.g[u][v], e);
        gr[e] = w[i] * ge;
        if constexpr (ACC) gr[e] = elem<V>(sl.old[u][v][i], e) + gr[e];
        const float q = ge * elem<V>(sl.r[u][v][i], e);  // exact in the normal range
        acc[i] = acc[i] + q;
      }
      store_vec<V, kNontemporal>(gr_row[i], h, pack<V>(gr));
    }
  }
}

// Grid: (ceil(T / tokens_per_block), n / S) blocks of exactly 256 threads,
// n the expansion rate (2, 4 or 8 residual streams per token). Block (b, j)
// handles streams S*j .. S*j + S-1 of tokens b*tokens_per_block ..
// (b+1)*tokens_per_block - 1, one token after the other. The fixed order is
// defined per (token, stream), so splitting a token's streams over blocks
// changes no bit and needs no communication between blocks: S = 4 keeps a
// 4-stream token in one block (grad_out read once), S = 1 gives four times
// as many blocks for short batches.
//
// Lane l (= threadIdx.x) is accumulator lane l of the fixed order: it visits
// groups k = l, l + 256, l + 512, ... (group k = hidden elements 8k .. 8k+7),
// U of them in flight at a time, and for each element adds grad_out*residual_i
// to its accumulator i in ascending h. It also writes grad_residual for every
// element it visits (ACC: adds the product to the stored gradient in fp32 and
// rounds the sum once). Then each wave halves its 64 accumulators with
// offsets 32..1 and the four wave results meet in LDS as (y0+y2)+(y1+y3).
// V elements are moved per access; V divides 8 and H, so a group is 8/V
// accesses (fewer for a short last group).
//
// At most 128 VGPRs (4 waves per SIMD), so that 4 blocks fit on a CU: the
// policy uses this layout for batches below 544 rows (136 tokens at
// n = 4), which are then resident at once.
//
// As in the row layout, the arguments the first loads need come first (the
// build preloads them into scalar registers); pre and grad_pre follow.
template <int V, int U, int S, bool ACC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void hagg_bwd_kernel(
    const uint16_t* __restrict__ residual, const uint16_t* __restrict__ grad_out,
    uint16_t* __restrict__ grad_residual, int64_t H, int64_t T, uint32_t ngroups,
    int32_t tokens_per_block, int32_t n, const float* __restrict__ pre,
    float* __restrict__ grad_pre) {
  __shared__ float wave_sum[4][S];  // [wave][stream of this block]

  const int lane = threadIdx.x;
  const int wave = lane >> 6;
  const int i0 = static_cast<int>(blockIdx.y) * S;  // first stream of this block

  for (int32_t tt = 0; tt < tokens_per_block; ++tt) {
    const int64_t t = static_cast<int64_t>(blockIdx.x) * tokens_per_block + tt;
    if (t >= T) break;  // uniform across the block

    // One resource per row: the token's grad_out row and the block's S
    // residual and grad_residual rows (2H bytes each). Groups past the end of
    // the row (k >= ngroups) and elements past H of a short last group read 0
    // and their stores are dropped, so the loop has no per-group branch: a
    // zero element adds +0 * +0 = +0 to an accumulator, which leaves it
    // bit-unchanged (an accumulator that starts at +0 is never -0 under
    // round-to-nearest), and its grad_residual store falls outside the row.
    const Rsrc g_row = make_rsrc(grad_out + t * H, 2 * H);
    Rsrc r_row[S], gr_row[S];
#pragma unroll
    for (int i = 0; i < S; ++i) {
      r_row[i] = make_rsrc(residual + (t * n + i0 + i) * H, 2 * H);
      gr_row[i] = make_rsrc(grad_residual + (t * n + i0 + i) * H, 2 * H);
    }

    float acc[S];
#pragma unroll
    for (int i = 0; i < S; ++i) acc[i] = 0.0f;

    // Lane l visits groups l, l + 256, l + 512, ... in that order, U of them
    // per round, through a ring of U register slots: slot u holds the group
    // of round j at position u, and is refilled with its group of round j+1
    // as soon as it has been consumed, so loads stay in flight while earlier
    // groups are computed and stored. The round count is taken from the
    // wave's first lane (the lanes of a wave differ by less than 64 groups),
    // so it is wave-uniform; a lane with fewer groups meets only zeros in its
    // last round.
    BwdSlots<V, U, S, ACC> sl;
    const uint32_t wave_first = __builtin_amdgcn_readfirstlane(lane & ~63u);
    const uint32_t step = kLanes * U;
    const uint32_t rounds = wave_first < ngroups ? (ngroups - wave_first + step - 1) / step : 0;
    if (rounds > 0) {
#pragma unroll
      for (int u = 0; u < U; ++u) bwd_issue(sl, u, lane + u * kLanes, g_row, r_row, gr_row);
      __builtin_amdgcn_sched_barrier(0);
      // The token's weights, read once the ring's first loads are out.
      const float* p = pre + n * t + i0;
      float w[S];
#pragma unroll
      for (int i = 0; i < S; ++i) w[i] = p[i];
      for (uint32_t j = 0; j + 1 < rounds; ++j) {
        const uint32_t k0 = lane + j * step;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          bwd_consume(sl, u, k0 + u * kLanes, w, acc, gr_row);
          bwd_issue(sl, u, k0 + step + u * kLanes, g_row, r_row, gr_row);
        }
      }
      const uint32_t k0 = lane + (rounds - 1) * step;
#pragma unroll
      for (int u = 0; u < U; ++u) bwd_consume(sl, u, k0 + u * kLanes, w, acc, gr_row);
    }

    // Wave stage: x[j] = x[j] + x[j + off] for off = 32, 16, 8, 4, 2, 1.
    // Lanes j >= off compute values nobody reads.
#pragma unroll
    for (int i = 0; i < S; ++i) acc[i] = acc[i] + from_lane_plus<32>(acc[i]);
#pragma unroll
    for (int i = 0; i < S; ++i) acc[i] = acc[i] + from_lane_plus<16>(acc[i]);
#pragma unroll
    for (int i = 0; i < S; ++i) acc[i] = acc[i] + from_lane_plus<8>(acc[i]);
#pragma unroll
    for (int i = 0; i < S; ++i) acc[i] = acc[i] + from_lane_plus<4>(acc[i]);
#pragma unroll
    for (int i = 0; i < S; ++i) acc[i] = acc[i] + from_lane_plus<2>(acc[i]);
#pragma unroll
    for (int i = 0; i < S; ++i) acc[i] = acc[i] + from_lane_plus<1>(acc[i]);
    if ((lane & 63) == 0) {
#pragma unroll
      for (int i = 0; i < S; ++i) wave_sum[wave][i] = acc[i];
    }
    __syncthreads();
    if (lane < S) {
      const float y02 = wave_sum[0][lane] + wave_sum[2][lane];
      const float y13 = wave_sum[1][lane] + wave_sum[3][lane];
      grad_pre[n * t + i0 + lane] = y02 + y13;
    }
    __syncthreads();  // wave_sum is reused by the next token
  }
}

// Row layout of the backward: one wave per (token, stream) row.
//
// Grid: ceil(T*n / R) blocks of 64*R threads (R rows per block, R = 1, 2, 4
// or 8); wave p of block b owns row q = R*b + p of the flattened [T, n] index,
// i.e. token q / n, stream q % n, and streams that whole row: grad_out row
// (shared by the n waves of a token, loaded with the default cache policy so
// the other waves find it in cache), residual row and grad_residual row.
//
// The fixed order is unchanged, only its lanes are laid out differently:
// physical lane j holds accumulator lanes j, j+64, j+128 and j+192 of the
// 256 (one accumulator each, acc[m] for lane j + 64m). Group k belongs to
// accumulator lane k mod 256, which is physical lane k mod 64 with
// m = (k / 64) mod 4; so lane j visits its groups k = j + 64c in ascending
// c ("chunk" c, one 1-KiB load per row for V = 8) and adds chunk c into
// acc[c mod 4] - each accumulator lane still sees its groups in ascending
// order. The wave stage of accumulator wave m is the halving tree over the
// 64 physical lanes on acc[m]; lane 0 then holds all four wave results and
// combines them as (y0+y2)+(y1+y3). No LDS, no barrier.
//
// Chunks pass through a ring of B register slots (B a multiple of 4, so a
// slot's accumulator index is a constant): slot b is refilled with chunk
// c + B as soon as chunk c has been consumed. Chunks past the end of the
// row read zeros and their stores are dropped (buffer range checks).
template <int V, int B, bool ACC>
struct RowSlots {
  typedef typename Vec<V>::type VT;
  static constexpr int NV = kGroup / V;
  VT g[B][NV];
  VT r[B][NV];
  VT old[ACC ? B : 1][NV];
};

template <int V, int B, bool ACC>
__device__ __forceinline__ void rows_issue(RowSlots<V, B, ACC>& sl, int b, uint32_t k, Rsrc g_row,
                                           Rsrc r_row, Rsrc gr_row) {
#pragma unroll
  for (int v = 0; v < RowSlots<V, B, ACC>::NV; ++v) {
    const uint32_t h = k * kGroup + v * V;
    sl.g[b][v] = load_vec<V, kCached>(g_row, h, 0);
    sl.r[b][v] = load_vec<V>(r_row, h, 0);
    if constexpr (ACC) sl.old[b][v] = load_vec<V>(gr_row, h, 0);
  }
}

template <int V, int B, bool ACC>
__device__ __forceinline__ void rows_consume(RowSlots<V, B, ACC>& sl, int b, uint32_t k, float w,
                                             float& acc, Rsrc gr_row) {
#pragma unroll
  for (int v = 0; v < RowSlots<V, B, ACC>::NV; ++v) {
    const uint32_t h = k * kGroup + v * V;
    float gr[V];
#pragma unroll
    for (int e = 0; e < V; ++e) {
      const float ge = elem<V>(sl.g[b][v], e);
      gr[e] = w * ge;
      if constexpr (ACC) gr[e] = elem<V>(sl.old[b][v], e) + gr[e];
      const float q = ge * elem<V>(sl.r[b][v], e);  // exact in the normal range
      acc = acc + q;
    }
    store_vec<V, kNontemporal>(gr_row, h, pack<V>(gr));
  }
}

//
// C > 0: the row has exactly C chunks (a compile-time count, for rows of up
// to 16 chunks): the chunk loop is unrolled completely and visits exactly
// those C chunks, refilling slot c mod B with chunk c + B only while that
// chunk exists. C == 0: any length, with a loop over rounds of B chunks; the
// last round may visit chunks past the end of the row, which read zeros
// (adding +0 leaves the accumulators unchanged) and whose stores are
// dropped: no memory traffic, but their instructions still run (at H = 7168,
// 16 chunk slots for 14 chunks; the exact count measured 1.2-1.7% faster
// at T = 1024 to 8192).
//
// PROGRESS (exact-count rows only): the wave starts at issue priority 3 and
// lowers it by one each time it has consumed another quarter of its row's
// chunks (s_setprio; the priority among the waves of a SIMD). Without it
// all waves share one priority and a CU serves its waves oldest first, so
// a launch whose blocks are all resident at once finishes in a tail where
// only each CU's youngest waves still stream; with it the waves of such a
// launch progress together (measured at H = 7168: T = 512 12.10 -> 11.35
// us, T = 1024 22.02 -> 21.24 us; the accumulating form, with a third
// stream of loads, gets 3-6% slower instead). When blocks start in several
// generations, the new waves would outrank the old ones and delay the
// slots they free (T = 2048 +14%, T = 8192 +12%), so the host uses it only
// when every block of the launch can be resident at once. The choice is a
// template argument, not a runtime branch: a branch joining inside the
// ring makes the compiler wait for every outstanding access at each later
// chunk.
//
// The arguments a wave needs before its first loads come first, so that the
// build's kernel-argument preloading places them in scalar registers: no
// argument load, block-size read or 64-bit division precedes the ring's
// first requests (n is a power of two, passed as log2n; rows_per_block is
// the block's wave count).
template <int V, int B, bool ACC, int C, bool PROGRESS>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4))) void hagg_bwd_rows_kernel(
    const uint16_t* __restrict__ residual, const uint16_t* __restrict__ grad_out,
    uint16_t* __restrict__ grad_residual, int64_t H, int64_t rows, uint32_t log2n,
    uint32_t rows_per_block, uint32_t ngroups, const float* __restrict__ pre,
    float* __restrict__ grad_pre) {
  static_assert(B % 4 == 0, "ring size must be a multiple of 4");
  static_assert(!PROGRESS || C > 0, "progress priority needs the exact chunk count");
  const uint32_t lane = threadIdx.x & 63;
  const int64_t q = static_cast<int64_t>(blockIdx.x) * rows_per_block +
                    __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (q >= rows) return;  // the whole wave
  const int64_t t = q >> log2n;
  const Rsrc g_row = make_rsrc(grad_out + t * H, 2 * H);
  const Rsrc r_row = make_rsrc(residual + q * H, 2 * H);
  const Rsrc gr_row = make_rsrc(grad_residual + q * H, 2 * H);

  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  RowSlots<V, B, ACC> sl;
  if constexpr (C > 0) {
    // The scheduling barriers keep the loads in chunk order (the compiler
    // would otherwise be free to issue later chunks first, and the first
    // chunk's arithmetic would wait for most of the ring).
    constexpr int kFirst = C < B ? C : B;
    if constexpr (PROGRESS) __builtin_amdgcn_s_setprio(3);
#pragma unroll
    for (int b = 0; b < kFirst; ++b) {
      rows_issue(sl, b, lane + 64 * b, g_row, r_row, gr_row);
      __builtin_amdgcn_sched_barrier(0);
    }
    const float w = pre[q];  // pre[t, q mod n], read once the ring's first loads are out
#pragma unroll
    for (int c = 0; c < C; ++c) {
      rows_consume(sl, c % B, lane + 64 * c, w, acc[c & 3], gr_row);
      if (c + B < C) rows_issue(sl, c % B, lane + 64 * (c + B), g_row, r_row, gr_row);
      if constexpr (PROGRESS) {
        // Quarters of the row consumed before and after chunk c, capped at 3
        // (constants once the loop is unrolled); priority 3 - quarters.
        const int before = 4 * c / C < 3 ? 4 * c / C : 3;
        const int after = 4 * (c + 1) / C < 3 ? 4 * (c + 1) / C : 3;
        if (after != before) {
          if (after == 1) __builtin_amdgcn_s_setprio(2);
          if (after == 2) __builtin_amdgcn_s_setprio(1);
          if (after == 3) __builtin_amdgcn_s_setprio(0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    const uint32_t chunks = (ngroups + 63) / 64;
    const uint32_t rounds = (chunks + B - 1) / B;
#pragma unroll
    for (int b = 0; b < B; ++b) {
      rows_issue(sl, b, lane + 64 * b, g_row, r_row, gr_row);
      __builtin_amdgcn_sched_barrier(0);
    }
    const float w = pre[q];
    for (uint32_t j = 0; j + 1 < rounds; ++j) {
      const uint32_t k0 = lane + 64 * B * j;
#pragma unroll
      for (int b = 0; b < B; ++b) {
        rows_consume(sl, b, k0 + 64 * b, w, acc[b & 3], gr_row);
        rows_issue(sl, b, k0 + 64 * (B + b), g_row, r_row, gr_row);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    const uint32_t k0 = lane + 64 * B * (rounds - 1);
#pragma unroll
    for (int b = 0; b < B; ++b) rows_consume(sl, b, k0 + 64 * b, w, acc[b & 3], gr_row);
  }

  // Wave stage for each accumulator wave m, then the block stage in lane 0.
#pragma unroll
  for (int m = 0; m < 4; ++m) acc[m] = acc[m] + from_lane_plus<32>(acc[m]);
#pragma unroll
  for (int m = 0; m < 4; ++m) acc[m] = acc[m] + from_lane_plus<16>(acc[m]);
#pragma unroll
  for (int m = 0; m < 4; ++m) acc[m] = acc[m] + from_lane_plus<8>(acc[m]);
#pragma unroll
  for (int m = 0; m < 4; ++m) acc[m] = acc[m] + from_lane_plus<4>(acc[m]);
#pragma unroll
  for (int m = 0; m < 4; ++m) acc[m] = acc[m] + from_lane_plus<2>(acc[m]);
#pragma unroll
  for (int m = 0; m < 4; ++m) acc[m] = acc[m] + from_lane_plus<1>(acc[m]);
  if (lane == 0) {
    const float y02 = acc[0] + acc[2];
    const float y13 = acc[1] + acc[3];
    grad_pre[q] = y02 + y13;
  }
}

// ---------------------------------------------------------------------------
// Host side: error text, validation, launch policy
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

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
  const char* name;
};

bool overlap(const Range& a, const Range& b) { return a.lo < b.hi && b.lo < a.hi; }

// Byte sizes of every tensor, or an error if T, n, H or the sizes are invalid.
struct Sizes {
  int64_t res_bytes, pre_bytes, row_bytes;  // [T,n,H] bf16, [T,n] fp32, [T,H] bf16
};

mhc_status check_sizes(int64_t T, int32_t n, int64_t H, Sizes* s) {
  if (n != 2 && n != 4 && n != 8)
    return fail(MHC_ERROR_INVALID_VALUE, "the expansion rate n must be 2, 4 or 8 (got %d)", n);
  if (T < 0) return fail(MHC_ERROR_INVALID_VALUE, "T must be >= 0 (got %lld)", (long long)T);
  if (H < 1 || H > MHC_MAX_H)
    return fail(MHC_ERROR_INVALID_VALUE, "H must be in [1, %lld] (got %lld)",
                (long long)MHC_MAX_H, (long long)H);
  // 2*n*T*H must fit int64 (residual bytes).
  if (T > INT64_MAX / (2 * n) / H)
    return fail(MHC_ERROR_INVALID_VALUE, "T*H too large: byte counts overflow int64");
  s->res_bytes = 2 * n * T * H;
  s->row_bytes = 2 * T * H;
  s->pre_bytes = 4 * n * T;
  return ok();
}

mhc_status check_ptr(const void* p, int64_t align, const char* name) {
  if (p == nullptr) return fail(MHC_ERROR_INVALID_VALUE, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(p) % align != 0)
    return fail(MHC_ERROR_INVALID_VALUE, "%s is not %lld-byte aligned", name, (long long)align);
  return ok();
}

Range range(const void* p, int64_t bytes, const char* name) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + static_cast<uintptr_t>(bytes), name};
}

mhc_status check_disjoint(const Range* outs, int nout, const Range* ins, int nin) {
  for (int a = 0; a < nout; ++a) {
    for (int b = 0; b < nin; ++b)
      if (overlap(outs[a], ins[b]))
        return fail(MHC_ERROR_ALIASING, "output %s overlaps input %s", outs[a].name, ins[b].name);
    for (int b = a + 1; b < nout; ++b)
      if (overlap(outs[a], outs[b]))
        return fail(MHC_ERROR_ALIASING, "output %s overlaps output %s", outs[a].name, outs[b].name);
  }
  return ok();
}

// Widest V in {8,4,2,1} that divides H and keeps every listed bf16 buffer's
// rows V-aligned.
int widest_vec(int64_t H, const void* const* bufs, int nbufs) {
  for (int V = 8; V > 1; V >>= 1) {
    if (H % V != 0) continue;
    bool aligned = true;
    for (int i = 0; i < nbufs; ++i)
      if (reinterpret_cast<uintptr_t>(bufs[i]) % (2 * V) != 0) aligned = false;
    if (aligned) return V;
  }
  return 1;
}

bool vec_allowed(int V, int64_t H, const void* const* bufs, int nbufs) {
  if (V != 1 && V != 2 && V != 4 && V != 8) return false;
  if (H % V != 0) return false;
  for (int i = 0; i < nbufs; ++i)
    if (reinterpret_cast<uintptr_t>(bufs[i]) % (2 * V) != 0) return false;
  return true;
}

// One dispatch covers at most 2^31 work-items (the AQL packet's grid size is a
// 32-bit work-item count); larger problems are split over whole tokens.
constexpr int64_t kMaxLaunchThreads = int64_t(1) << 31;
constexpr int64_t kMaxGridY = 65535;
// Backward layout and streams per block by batch length (see plan_bwd).
constexpr int64_t kTwoStreamsFromT = 128;
constexpr int64_t kFourStreamsFromT = 512;
// The row layout from this many rows (tokens x streams) per call on: it has
// one wave per row, the split layout 4 per block of S streams, so short
// batches keep more CUs busy split. Measured at H = 7168: split faster at
// 512 rows for n = 2, 4 and 8 (by 6-10%); rows faster or equal from 544 rows
// at n = 4 and from 576 at n = 2 and 8 (at n = 4 except at 320-384 tokens,
// by 1-7%).
constexpr int64_t kRowsFromRows = 544;
// Row-layout rows of at most this many chunks (64 groups of 8 elements each:
// H <= 8192) use a kernel compiled for their exact chunk count (16-byte
// accesses only, the common case).
constexpr int kMaxFixedChunks = 16;

// Largest forward batch UPT in {1, 2, 4} whose loaded data (N rows, each
// access max(V/2, 1) registers) fits 64 VGPRs, within the 128-VGPR budget of
// a 1024-thread block.
constexpr int fwd_max_upt(int V, int N) {
  const int per_unit = N * (V >= 2 ? V / 2 : 1);
  return 4 * per_unit <= 64 ? 4 : (2 * per_unit <= 64 ? 2 : 1);
}

struct FwdPlan {
  int V, block, upt, n;
  uint32_t blocks_per_token;
  int64_t tokens_per_launch, total_blocks;
};

mhc_status plan_fwd(const uint16_t* residual, const uint16_t* out, int64_t T, int32_t n,
                    int64_t H, const mhc_launch* ov, FwdPlan* pl) {
  const void* bufs[2] = {residual, out};
  int V = widest_vec(H, bufs, 2);
  if (ov && ov->vec_width != 0) {
    if (!vec_allowed(ov->vec_width, H, bufs, 2))
      return fail(MHC_ERROR_INVALID_VALUE,
                  "vec_width %d not allowed for H=%lld and the buffers' alignment",
                  ov->vec_width, (long long)H);
    V = ov->vec_width;
  }
  if (ov && (ov->tokens_per_block != 0 || ov->streams_per_block != 0 || ov->layout != 0 ||
             ov->wave_priority != 0))
    return fail(MHC_ERROR_INVALID_VALUE,
                "tokens_per_block, streams_per_block, layout and wave_priority are backward-only "
                "fields");
  const int64_t upt_units = H / V;  // units per token
  const int max_upt = fwd_max_upt(V, n);
  int upt = 1;
  if (ov && ov->units_per_thread != 0) {
    if (ov->units_per_thread != 1 && ov->units_per_thread != 2 && ov->units_per_thread != 4)
      return fail(MHC_ERROR_INVALID_VALUE, "units_per_thread must be 1, 2 or 4");
    upt = ov->units_per_thread;
    if (upt > max_upt)
      return fail(MHC_ERROR_INVALID_VALUE,
                  "units_per_thread %d exceeds the register budget (at most %d for vec_width "
                  "%d, n=%d)", upt, max_upt, V, n);
  }
  // One wave per block: on gfx950 the 64-thread shape measured fastest at
  // every bandwidth shape swept (T = 1024 and 8192, H = 7168), since the
  // most independent blocks give the workgroup dispatcher the most freedom
  // to spread the stream over 8 XCDs x 32 CUs; small problems gain from it
  // too (more CUs busy).
  int block = 64;
  if (ov && ov->block_threads != 0) {
    if (ov->block_threads < 64 || ov->block_threads > 1024 || ov->block_threads % 64 != 0)
      return fail(MHC_ERROR_INVALID_VALUE, "block_threads must be a multiple of 64 in [64, 1024]");
    block = ov->block_threads;
  }
  const int64_t span = static_cast<int64_t>(block) * upt;
  const int64_t bpt = (upt_units + span - 1) / span;
  pl->V = V;
  pl->block = block;
  pl->upt = upt;
  pl->n = n;
  pl->blocks_per_token = static_cast<uint32_t>(bpt);
  // Tokens run along the grid's y dimension, at most 65535 per launch, and a
  // launch stays within 2^31 work-items.
  int64_t tpl = kMaxLaunchThreads / (bpt * block);
  if (tpl > kMaxGridY) tpl = kMaxGridY;
  if (tpl < 1) tpl = 1;  // cannot happen for H <= MHC_MAX_H
  pl->tokens_per_launch = tpl;
  pl->total_blocks = T * bpt;
  return ok();
}

// Largest ring size U in {1, 2, 4} whose loaded data fits 88 VGPRs: per
// group NV = 8/V accesses of each of the 1 + S (+ S stored gradients when
// accumulating) rows, each access max(V/2, 1) registers. With the rest of
// the kernel (and the refill of a slot while the next is consumed) this
// stays under the 128-VGPR budget without spills.
constexpr int bwd_max_u(int V, int S, bool acc) {
  const int per_group = (kGroup / V) * (1 + (acc ? 2 : 1) * S) * (V >= 2 ? V / 2 : 1);
  return 4 * per_group <= 88 ? 4 : (2 * per_group <= 88 ? 2 : 1);
}

// Largest ring size B in {4, 8, 12} of the row layout whose loaded data fits
// 96 VGPRs: per chunk NV = 8/V accesses of the grad_out and residual rows
// (and the stored gradient when accumulating), each max(V/2, 1) registers.
// Scalar-width accesses (V = 1) hold one element per register and need
// widening temporaries, so their budget is 64; 0 means the row layout is not
// available for that shape (the split layout is used).
constexpr int rows_max_b(int V, bool acc) {
  const int per_chunk = (kGroup / V) * (acc ? 3 : 2) * (V >= 2 ? V / 2 : 1);
  const int budget = V == 1 ? 64 : 96;
  return 12 * per_chunk <= budget ? 12
         : 8 * per_chunk <= budget ? 8
         : 4 * per_chunk <= budget ? 4 : 0;
}

// Compute units of the current device, cached per device; 256 (every gfx950
// part) when no device can be queried, as when a plan is computed on a host
// without a GPU.
int64_t compute_units() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < kMaxDevices) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return 256;
  if (dev < kMaxDevices) cached[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// Waves every CU holds of any row-layout instance: the kernels are built for
// at least 4 waves per SIMD (amdgpu_waves_per_eu), 4 SIMDs per CU.
constexpr int64_t kResidentRowsPerCU = 16;

struct BwdPlan {
  int layout;  // MHC_BWD_SPLIT or MHC_BWD_ROWS
  int V, U, S, tpb, n;
  int rows_per_block;  // row layout
  int fixed_chunks;    // row layout: the row's chunk count if compiled in, else 0
  bool progress;       // row layout: issue priority by progress (PROGRESS instances)
  bool acc;
  int64_t ngroups, blocks_per_launch, total_blocks;
};

mhc_status plan_bwd(const uint16_t* residual, const uint16_t* grad_out,
                    const uint16_t* grad_residual, int64_t T, int32_t n, int64_t H, bool acc,
                    const mhc_launch* ov, BwdPlan* pl) {
  const void* bufs[3] = {residual, grad_out, grad_residual};
  int V = widest_vec(H, bufs, 3);
  if (ov && ov->vec_width != 0) {
    if (!vec_allowed(ov->vec_width, H, bufs, 3))
      return fail(MHC_ERROR_INVALID_VALUE,
                  "vec_width %d not allowed for H=%lld and the buffers' alignment",
                  ov->vec_width, (long long)H);
    V = ov->vec_width;
  }
  // Row layout from kRowsFromRows rows on, unless a split-layout field is set.
  const bool rows_ok = rows_max_b(V, acc) > 0;
  const bool split_fields = ov && (ov->tokens_per_block != 0 || ov->streams_per_block != 0);
  int layout =
      T * n >= kRowsFromRows && rows_ok && !split_fields ? MHC_BWD_ROWS : MHC_BWD_SPLIT;
  if (ov && ov->layout != 0) {
    if (ov->layout != MHC_BWD_SPLIT && ov->layout != MHC_BWD_ROWS)
      return fail(MHC_ERROR_INVALID_VALUE, "backward layout must be 0, %d or %d", MHC_BWD_SPLIT,
                  MHC_BWD_ROWS);
    if (ov->layout == MHC_BWD_ROWS && !rows_ok)
      return fail(MHC_ERROR_INVALID_VALUE,
                  "the row layout exceeds the register budget at vec_width %d%s", V,
                  acc ? ", accumulating" : "");
    layout = ov->layout;
  }
  pl->layout = layout;
  pl->V = V;
  pl->n = n;
  pl->acc = acc;
  pl->ngroups = (H + kGroup - 1) / kGroup;
  if (layout == MHC_BWD_ROWS) {
    // One wave per (token, stream) row, 4 rows per block: a token's waves
    // (or half of them at n = 8) run on one CU and share its grad_out row
    // through the cache. Measured: 1 or 2 rows per block slower at every n;
    // at n = 8, 4 rows 3-5% faster than 8 (T = 512, 1024, H = 7168).
    int R = 4;
    if (ov && ov->block_threads != 0) {
      if (ov->block_threads != 64 && ov->block_threads != 128 && ov->block_threads != 256 &&
          ov->block_threads != 512)
        return fail(MHC_ERROR_INVALID_VALUE,
                    "row-layout backward block_threads must be 0, 64, 128, 256 or 512");
      R = ov->block_threads / 64;
    }
    if (ov && (ov->tokens_per_block != 0 || ov->streams_per_block != 0))
      return fail(MHC_ERROR_INVALID_VALUE,
                  "tokens_per_block and streams_per_block belong to the split layout");
    // Ring size, fewer where the register budget requires: 12 chunks in
    // flight for rows compiled for their exact chunk count (the whole row
    // up to H = 6144; measured at H = 7168 against 8: 22.01 / 41.38 / 171.4
    // us against 22.09 / 41.69 / 174.2 at T = 1024 / 2048 / 8192), 8 for the
    // looping kernel, whose last round would visit 12 slots for any
    // remainder (8 measured fastest there at T = 512 to 2048).
    const int max_b = rows_max_b(V, acc);
    const int64_t row_chunks = (pl->ngroups + 63) / 64;
    const bool exact = V == 8 && row_chunks <= kMaxFixedChunks;
    const int want_b = exact ? 12 : 8;
    int B = max_b < want_b ? max_b : want_b;
    if (ov && ov->units_per_thread != 0) {
      if (ov->units_per_thread != 4 && ov->units_per_thread != 8 && ov->units_per_thread != 12)
        return fail(MHC_ERROR_INVALID_VALUE, "row-layout units_per_thread must be 4, 8 or 12");
      B = ov->units_per_thread;
      if (B > max_b)
        return fail(MHC_ERROR_INVALID_VALUE,
                    "units_per_thread %d exceeds the register budget (at most %d for vec_width "
                    "%d%s)",
                    B, max_b, V, acc ? ", accumulating" : "");
    }
    pl->U = B;
    pl->S = 0;
    pl->tpb = 0;
    pl->rows_per_block = R;
    const int64_t chunks = (pl->ngroups + 63) / 64;
    pl->fixed_chunks = V == 8 && chunks <= kMaxFixedChunks ? static_cast<int>(chunks) : 0;
    // Issue priority by progress when every row of the call has a wave slot
    // from the start (hagg_bwd_rows_kernel, PROGRESS): at n = 4 and 256 CUs,
    // up to T = 1024. Not for the accumulating backward, which it slows
    // (H = 7168, T * n = 2048 to 4096 rows, n = 2, 4, 8: 3.5-6% faster
    // written, 3-6% slower accumulating).
    bool progress = !acc && pl->fixed_chunks > 0 && T * n <= kResidentRowsPerCU * compute_units();
    if (ov && ov->wave_priority != 0) {
      if (ov->wave_priority != MHC_PRIO_FLAT && ov->wave_priority != MHC_PRIO_PROGRESS)
        return fail(MHC_ERROR_INVALID_VALUE, "wave_priority must be 0, %d or %d", MHC_PRIO_FLAT,
                    MHC_PRIO_PROGRESS);
      if (ov->wave_priority == MHC_PRIO_PROGRESS && pl->fixed_chunks == 0)
        return fail(MHC_ERROR_INVALID_VALUE,
                    "wave_priority %d needs rows of at most %d chunks of 16-byte accesses "
                    "(vec_width 8, H <= %d)",
                    MHC_PRIO_PROGRESS, kMaxFixedChunks, kMaxFixedChunks * 64 * kGroup);
      progress = ov->wave_priority == MHC_PRIO_PROGRESS;
    }
    pl->progress = progress;
    // Whole tokens per launch: blocks_per_launch * R rows is a multiple of n
    // (R and n are powers of two, n <= 8, and blocks_per_launch is a
    // multiple of 8).
    pl->blocks_per_launch = kMaxLaunchThreads / (64 * R);
    pl->total_blocks = (T * n + R - 1) / R;
    return ok();
  }
  if (ov && ov->block_threads != 0 && ov->block_threads != kLanes)
    return fail(MHC_ERROR_INVALID_VALUE, "split-layout backward block_threads must be 0 or 256");
  if (ov && ov->wave_priority != 0 && ov->wave_priority != MHC_PRIO_FLAT)
    return fail(MHC_ERROR_INVALID_VALUE, "the split layout runs its waves at one priority "
                "(wave_priority 0 or %d)", MHC_PRIO_FLAT);
  // Streams per block: all of a token's streams (up to four) in one block
  // once there are enough tokens to cover the CUs (grad_out is then read once
  // per block); shorter batches spread each token over more blocks to use
  // more CUs. Thresholds measured at n = 4, H = 4096 and 7168 (T from 1 to
  // 2048).
  int S = T >= kFourStreamsFromT ? 4 : (T >= kTwoStreamsFromT ? 2 : 1);
  if (S > n) S = n;
  if (ov && ov->streams_per_block != 0) {
    if (ov->streams_per_block != 1 && ov->streams_per_block != 2 && ov->streams_per_block != 4)
      return fail(MHC_ERROR_INVALID_VALUE, "streams_per_block must be 1, 2 or 4");
    if (ov->streams_per_block > n)
      return fail(MHC_ERROR_INVALID_VALUE, "streams_per_block %d exceeds the %d streams",
                  ov->streams_per_block, n);
    S = ov->streams_per_block;
  }
  // Groups each lane loads before its arithmetic: as many as the register
  // budget allows, up to four (all of a lane's groups at H = 7168), so every
  // byte a lane needs is in flight at once while all blocks of a 1024-token
  // call stay resident; four measured fastest at T = 1024, 2048 and 8192.
  const int max_u = bwd_max_u(V, S, acc);
  int U = max_u;
  if (ov && ov->units_per_thread != 0) {
    if (ov->units_per_thread != 1 && ov->units_per_thread != 2 && ov->units_per_thread != 4)
      return fail(MHC_ERROR_INVALID_VALUE, "units_per_thread must be 1, 2 or 4");
    U = ov->units_per_thread;
    if (U > max_u)
      return fail(MHC_ERROR_INVALID_VALUE,
                  "units_per_thread %d exceeds the register budget (at most %d for vec_width "
                  "%d, %d streams per block%s)",
                  U, max_u, V, S, acc ? ", accumulating" : "");
  }
  int tpb = 1;
  if (ov && ov->tokens_per_block != 0) {
    if (ov->tokens_per_block < 1 || ov->tokens_per_block > 4096)
      return fail(MHC_ERROR_INVALID_VALUE, "tokens_per_block must be in [1, 4096]");
    tpb = ov->tokens_per_block;
  }
  pl->U = U;
  pl->S = S;
  pl->tpb = tpb;
  pl->rows_per_block = 0;
  pl->fixed_chunks = 0;
  pl->progress = false;
  pl->blocks_per_launch = kMaxLaunchThreads / kLanes / (n / S);
  pl->total_blocks = (T + tpb - 1) / tpb * (n / S);
  return ok();
}

mhc_status validate_fwd(const uint16_t* residual, const float* pre, const uint16_t* out,
                        int64_t T, int32_t n, int64_t H) {
  Sizes s;
  mhc_status st = check_sizes(T, n, H, &s);
  if (st != MHC_SUCCESS || T == 0) return st;
  if ((st = check_ptr(residual, 2, "residual")) != MHC_SUCCESS) return st;
  if ((st = check_ptr(pre, 4, "pre")) != MHC_SUCCESS) return st;
  if ((st = check_ptr(out, 2, "out")) != MHC_SUCCESS) return st;
  const Range ins[2] = {range(residual, s.res_bytes, "residual"), range(pre, s.pre_bytes, "pre")};
  const Range outs[1] = {range(out, s.row_bytes, "out")};
  return check_disjoint(outs, 1, ins, 2);
}

mhc_status validate_bwd(const uint16_t* residual, const float* pre, const uint16_t* grad_out,
                        const uint16_t* grad_residual, const float* grad_pre, int64_t T,
                        int32_t n, int64_t H) {
  Sizes s;
  mhc_status st = check_sizes(T, n, H, &s);
  if (st != MHC_SUCCESS || T == 0) return st;
  if ((st = check_ptr(residual, 2, "residual")) != MHC_SUCCESS) return st;
  if ((st = check_ptr(pre, 4, "pre")) != MHC_SUCCESS) return st;
  if ((st = check_ptr(grad_out, 2, "grad_out")) != MHC_SUCCESS) return st;
  if ((st = check_ptr(grad_residual, 2, "grad_residual")) != MHC_SUCCESS) return st;
  if ((st = check_ptr(grad_pre, 4, "grad_pre")) != MHC_SUCCESS) return st;
  const Range ins[3] = {range(residual, s.res_bytes, "residual"), range(pre, s.pre_bytes, "pre"),
                        range(grad_out, s.row_bytes, "grad_out")};
  const Range outs[2] = {range(grad_residual, s.res_bytes, "grad_residual"),
                         range(grad_pre, s.pre_bytes, "grad_pre")};
  return check_disjoint(outs, 2, ins, 3);
}

// The status of one launch (the value hipExtLaunchKernel returned for it).
mhc_status launch_status(hipError_t e, const char* what) {
  if (e != hipSuccess)
    return fail(MHC_ERROR_HIP, "%s launch failed: %s (%s)", what, hipGetErrorName(e),
                hipGetErrorString(e));
  return ok();
}

// Kernel launches go through launch_kernel (mhc_launch.h): each returns the
// status of its own launch, and a caller's timing events can be attached to
// the dispatch itself (the start event takes the dispatch's start timestamp
// and the stop event its end timestamp, with no extra marker packets between
// kernels). Null events give a plain launch.
struct Events {
  hipEvent_t start, stop;
};

template <int V, int UPT, int N>
hipError_t launch_fwd_t(const FwdPlan& pl, const uint16_t* residual, const float* pre, uint16_t* out,
                        int64_t tokens, int64_t H, hipStream_t stream, Events ev) {
  return launch_kernel(hagg_fwd_kernel<V, UPT, N>,
                       dim3(pl.blocks_per_token, static_cast<uint32_t>(tokens)), dim3(pl.block),
                       stream, ev.start, ev.stop, residual, pre, out, H,
                       static_cast<uint32_t>(pl.block));
}

// Instantiates only the batches the register budget allows (the plan never
// asks for more).
template <int V, int N>
hipError_t launch_fwd_n(const FwdPlan& pl, const uint16_t* residual, const float* pre, uint16_t* out,
                        int64_t tokens, int64_t H, hipStream_t stream, Events ev) {
  constexpr int kMax = fwd_max_upt(V, N);
  constexpr int kU2 = kMax < 2 ? kMax : 2;
  switch (pl.upt) {
    case 1: return launch_fwd_t<V, 1, N>(pl, residual, pre, out, tokens, H, stream, ev);
    case 2: return launch_fwd_t<V, kU2, N>(pl, residual, pre, out, tokens, H, stream, ev);
    default: return launch_fwd_t<V, kMax, N>(pl, residual, pre, out, tokens, H, stream, ev);
  }
}

template <int V>
hipError_t launch_fwd_v(const FwdPlan& pl, const uint16_t* residual, const float* pre, uint16_t* out,
                        int64_t tokens, int64_t H, hipStream_t stream, Events ev) {
  switch (pl.n) {
    case 2: return launch_fwd_n<V, 2>(pl, residual, pre, out, tokens, H, stream, ev);
    case 8: return launch_fwd_n<V, 8>(pl, residual, pre, out, tokens, H, stream, ev);
    default: return launch_fwd_n<V, 4>(pl, residual, pre, out, tokens, H, stream, ev);
  }
}

template <int V, int U, int S, bool ACC>
hipError_t launch_bwd_t(const BwdPlan& pl, const uint16_t* residual, const float* pre,
                        const uint16_t* grad_out, uint16_t* grad_residual, float* grad_pre,
                        int64_t tokens, int64_t H, hipStream_t stream, Events ev) {
  const uint32_t blocks = static_cast<uint32_t>((tokens + pl.tpb - 1) / pl.tpb);
  return launch_kernel(hagg_bwd_kernel<V, U, S, ACC>, dim3(blocks, pl.n / S), dim3(kLanes), stream,
                       ev.start, ev.stop, residual, grad_out, grad_residual, H, tokens,
                       static_cast<uint32_t>(pl.ngroups), static_cast<int32_t>(pl.tpb),
                       static_cast<int32_t>(pl.n), pre, grad_pre);
}

// Instantiates only the batches the register budget allows (the plan never
// asks for more): U is clamped to bwd_max_u at compile time.
template <int V, int S, bool ACC>
hipError_t launch_bwd_s(const BwdPlan& pl, const uint16_t* residual, const float* pre,
                        const uint16_t* grad_out, uint16_t* grad_residual, float* grad_pre,
                        int64_t tokens, int64_t H, hipStream_t stream, Events ev) {
  constexpr int kMaxU = bwd_max_u(V, S, ACC);
  constexpr int kU2 = kMaxU < 2 ? kMaxU : 2;
  switch (pl.U) {
    case 1: return launch_bwd_t<V, 1, S, ACC>(pl, residual, pre, grad_out, grad_residual, grad_pre, tokens, H, stream, ev);
    case 2: return launch_bwd_t<V, kU2, S, ACC>(pl, residual, pre, grad_out, grad_residual, grad_pre, tokens, H, stream, ev);
    default: return launch_bwd_t<V, kMaxU, S, ACC>(pl, residual, pre, grad_out, grad_residual, grad_pre, tokens, H, stream, ev);
  }
}

template <int V, bool ACC>
hipError_t launch_bwd_a(const BwdPlan& pl, const uint16_t* residual, const float* pre,
                        const uint16_t* grad_out, uint16_t* grad_residual, float* grad_pre,
                        int64_t tokens, int64_t H, hipStream_t stream, Events ev) {
  switch (pl.S) {
    case 1: return launch_bwd_s<V, 1, ACC>(pl, residual, pre, grad_out, grad_residual, grad_pre, tokens, H, stream, ev);
    case 2: return launch_bwd_s<V, 2, ACC>(pl, residual, pre, grad_out, grad_residual, grad_pre, tokens, H, stream, ev);
    default: return launch_bwd_s<V, 4, ACC>(pl, residual, pre, grad_out, grad_residual, grad_pre, tokens, H, stream, ev);
  }
}

template <int V, int B, bool ACC, int C>
hipError_t launch_rows_c(const BwdPlan& pl, const uint16_t* residual, const float* pre,
                         const uint16_t* grad_out, uint16_t* grad_residual, float* grad_pre,
                         int64_t tokens, int64_t H, hipStream_t stream, Events ev) {
  const int64_t rows = tokens * pl.n;
  const uint32_t blocks = static_cast<uint32_t>((rows + pl.rows_per_block - 1) / pl.rows_per_block);
  const uint32_t log2n = static_cast<uint32_t>(__builtin_ctz(static_cast<unsigned>(pl.n)));
  if constexpr (C > 0) {
    if (pl.progress)
      return launch_kernel(hagg_bwd_rows_kernel<V, B, ACC, C, true>, dim3(blocks),
                           dim3(64 * pl.rows_per_block), stream, ev.start, ev.stop, residual,
                           grad_out, grad_residual, H, rows, log2n,
                           static_cast<uint32_t>(pl.rows_per_block),
                           static_cast<uint32_t>(pl.ngroups), pre, grad_pre);
  }
  return launch_kernel(hagg_bwd_rows_kernel<V, B, ACC, C, false>, dim3(blocks),
                       dim3(64 * pl.rows_per_block), stream, ev.start, ev.stop, residual, grad_out,
                       grad_residual, H, rows, log2n, static_cast<uint32_t>(pl.rows_per_block),
                       static_cast<uint32_t>(pl.ngroups), pre, grad_pre);
}

template <int V, int B, bool ACC>
hipError_t launch_rows_t(const BwdPlan& pl, const uint16_t* residual, const float* pre,
                         const uint16_t* grad_out, uint16_t* grad_residual, float* grad_pre,
                         int64_t tokens, int64_t H, hipStream_t stream, Events ev) {
#define MHC_ROWS_C(c) \
  case c: return launch_rows_c<V, B, ACC, c>(pl, residual, pre, grad_out, grad_residual, grad_pre, tokens, H, stream, ev)
  if constexpr (V == 8) {
    switch (pl.fixed_chunks) {
      MHC_ROWS_C(1); MHC_ROWS_C(2); MHC_ROWS_C(3); MHC_ROWS_C(4); MHC_ROWS_C(5); MHC_ROWS_C(6);
      MHC_ROWS_C(7); MHC_ROWS_C(8); MHC_ROWS_C(9); MHC_ROWS_C(10); MHC_ROWS_C(11);
      MHC_ROWS_C(12); MHC_ROWS_C(13); MHC_ROWS_C(14); MHC_ROWS_C(15); MHC_ROWS_C(16);
      default: break;
    }
  }
#undef MHC_ROWS_C
  return launch_rows_c<V, B, ACC, 0>(pl, residual, pre, grad_out, grad_residual, grad_pre, tokens,
                                     H, stream, ev);
}

// Instantiates only the ring sizes the register budget allows.
template <int V, bool ACC>
hipError_t launch_rows_a(const BwdPlan& pl, const uint16_t* residual, const float* pre,
                         const uint16_t* grad_out, uint16_t* grad_residual, float* grad_pre,
                         int64_t tokens, int64_t H, hipStream_t stream, Events ev) {
  constexpr int kMaxB = rows_max_b(V, ACC);
  if constexpr (kMaxB == 0) {
    return hipErrorInvalidValue;  // never planned: no row layout for this shape
  } else {
    constexpr int kB8 = kMaxB < 8 ? kMaxB : 8;
    switch (pl.U) {
      case 4: return launch_rows_t<V, 4, ACC>(pl, residual, pre, grad_out, grad_residual, grad_pre, tokens, H, stream, ev);
      case 8: return launch_rows_t<V, kB8, ACC>(pl, residual, pre, grad_out, grad_residual, grad_pre, tokens, H, stream, ev);
      default: return launch_rows_t<V, kMaxB, ACC>(pl, residual, pre, grad_out, grad_residual, grad_pre, tokens, H, stream, ev);
    }
  }
}

template <int V>
hipError_t launch_bwd_v(const BwdPlan& pl, const uint16_t* residual, const float* pre,
                        const uint16_t* grad_out, uint16_t* grad_residual, float* grad_pre,
                        int64_t tokens, int64_t H, hipStream_t stream, Events ev) {
  if (pl.layout == MHC_BWD_ROWS) {
    if (pl.acc)
      return launch_rows_a<V, true>(pl, residual, pre, grad_out, grad_residual, grad_pre, tokens, H, stream, ev);
    return launch_rows_a<V, false>(pl, residual, pre, grad_out, grad_residual, grad_pre, tokens, H, stream, ev);
  }
  if (pl.acc)
    return launch_bwd_a<V, true>(pl, residual, pre, grad_out, grad_residual, grad_pre, tokens, H, stream, ev);
  return launch_bwd_a<V, false>(pl, residual, pre, grad_out, grad_residual, grad_pre, tokens, H, stream, ev);
}

// Events of the i-th of n launches of one call: start on the first, stop on
// the last.
Events chunk_events(const Events& ev, int64_t first_token, int64_t next_token, int64_t T) {
  return Events{first_token == 0 ? ev.start : nullptr, next_token >= T ? ev.stop : nullptr};
}

// A call that launches nothing (T == 0) still records the caller's events,
// so their elapsed time is defined (zero work).
mhc_status record_empty(const Events& ev, hipStream_t s) {
  if (ev.start && hipEventRecord(ev.start, s) != hipSuccess)
    return fail(MHC_ERROR_HIP, "hipEventRecord(start) failed");
  if (ev.stop && hipEventRecord(ev.stop, s) != hipSuccess)
    return fail(MHC_ERROR_HIP, "hipEventRecord(stop) failed");
  return ok();
}

mhc_status run_fwd(const uint16_t* residual, const float* pre, uint16_t* out, int64_t T,
                   int32_t n, int64_t H, void* stream, const mhc_launch* launch, Events ev) {
  mhc_status st = validate_fwd(residual, pre, out, T, n, H);
  if (st != MHC_SUCCESS) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (T == 0) return record_empty(ev, s);
  FwdPlan pl;
  if ((st = plan_fwd(residual, out, T, n, H, launch, &pl)) != MHC_SUCCESS) return st;
  for (int64_t t0 = 0; t0 < T; t0 += pl.tokens_per_launch) {
    const int64_t m = (T - t0 < pl.tokens_per_launch) ? T - t0 : pl.tokens_per_launch;
    const Events e = chunk_events(ev, t0, t0 + m, T);
    const uint16_t* r = residual + t0 * n * H;
    const float* p = pre + n * t0;
    uint16_t* o = out + t0 * H;
    hipError_t err;
    switch (pl.V) {
      case 8: err = launch_fwd_v<8>(pl, r, p, o, m, H, s, e); break;
      case 4: err = launch_fwd_v<4>(pl, r, p, o, m, H, s, e); break;
      case 2: err = launch_fwd_v<2>(pl, r, p, o, m, H, s, e); break;
      default: err = launch_fwd_v<1>(pl, r, p, o, m, H, s, e); break;
    }
    if ((st = launch_status(err, "h_aggregate forward")) != MHC_SUCCESS) return st;
  }
  return ok();
}

mhc_status run_bwd(const uint16_t* residual, const float* pre, const uint16_t* grad_out,
                   uint16_t* grad_residual, float* grad_pre, int64_t T, int32_t n, int64_t H,
                   bool acc, void* stream, const mhc_launch* launch, Events ev) {
  mhc_status st = validate_bwd(residual, pre, grad_out, grad_residual, grad_pre, T, n, H);
  if (st != MHC_SUCCESS) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (T == 0) return record_empty(ev, s);
  BwdPlan pl;
  if ((st = plan_bwd(residual, grad_out, grad_residual, T, n, H, acc, launch, &pl)) != MHC_SUCCESS)
    return st;
  const int64_t tokens_per_launch = pl.layout == MHC_BWD_ROWS
                                        ? pl.blocks_per_launch * pl.rows_per_block / n
                                        : pl.blocks_per_launch * pl.tpb;
  for (int64_t t0 = 0; t0 < T; t0 += tokens_per_launch) {
    const int64_t m = (T - t0 < tokens_per_launch) ? T - t0 : tokens_per_launch;
    const Events e = chunk_events(ev, t0, t0 + m, T);
    const uint16_t* r = residual + t0 * n * H;
    const float* p = pre + n * t0;
    const uint16_t* g = grad_out + t0 * H;
    uint16_t* gr = grad_residual + t0 * n * H;
    float* gp = grad_pre + n * t0;
    hipError_t err;
    switch (pl.V) {
      case 8: err = launch_bwd_v<8>(pl, r, p, g, gr, gp, m, H, s, e); break;
      case 4: err = launch_bwd_v<4>(pl, r, p, g, gr, gp, m, H, s, e); break;
      case 2: err = launch_bwd_v<2>(pl, r, p, g, gr, gp, m, H, s, e); break;
      default: err = launch_bwd_v<1>(pl, r, p, g, gr, gp, m, H, s, e); break;
    }
    if ((st = launch_status(err, "h_aggregate backward")) != MHC_SUCCESS) return st;
  }
  return ok();
}

mhc_status plan_fwd_query(const uint16_t* residual, const float* pre, const uint16_t* out,
                          int64_t T, int32_t n, int64_t H, const mhc_launch* launch,
                          mhc_launch* plan, int64_t* grid_blocks) {
  mhc_status st = validate_fwd(residual, pre, out, T, n, H);
  if (st != MHC_SUCCESS) return st;
  FwdPlan pl;
  if ((st = plan_fwd(residual, out, T, n, H, launch, &pl)) != MHC_SUCCESS) return st;
  if (plan) *plan = mhc_launch{pl.block, pl.V, pl.upt, 0, 0, 0, 0};
  if (grid_blocks) *grid_blocks = pl.total_blocks;
  return ok();
}

mhc_status plan_bwd_query(const uint16_t* residual, const float* pre, const uint16_t* grad_out,
                          const uint16_t* grad_residual, const float* grad_pre, int64_t T,
                          int32_t n, int64_t H, bool acc, const mhc_launch* launch,
                          mhc_launch* plan, int64_t* grid_blocks) {
  mhc_status st = validate_bwd(residual, pre, grad_out, grad_residual, grad_pre, T, n, H);
  if (st != MHC_SUCCESS) return st;
  BwdPlan pl;
  if ((st = plan_bwd(residual, grad_out, grad_residual, T, n, H, acc, launch, &pl)) !=
      MHC_SUCCESS)
    return st;
  if (plan)
    *plan = pl.layout == MHC_BWD_ROWS
                ? mhc_launch{64 * pl.rows_per_block, pl.V, pl.U, 0, 0, MHC_BWD_ROWS,
                             pl.progress ? MHC_PRIO_PROGRESS : MHC_PRIO_FLAT}
                : mhc_launch{kLanes, pl.V, pl.U, pl.tpb, pl.S, MHC_BWD_SPLIT, MHC_PRIO_FLAT};
  if (grid_blocks) *grid_blocks = pl.total_blocks;
  return ok();
}

Events events(void* start_event, void* stop_event) {
  return Events{static_cast<hipEvent_t>(start_event), static_cast<hipEvent_t>(stop_event)};
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------

extern "C" {

int mhc_abi_version(void) { return MHC_ABI_VERSION; }

const char* mhc_status_string(mhc_status status) {
  switch (status) {
    case MHC_SUCCESS: return "MHC_SUCCESS";
    case MHC_ERROR_INVALID_VALUE: return "MHC_ERROR_INVALID_VALUE";
    case MHC_ERROR_ALIASING: return "MHC_ERROR_ALIASING";
    case MHC_ERROR_HIP: return "MHC_ERROR_HIP";
  }
  return "MHC_ERROR_UNKNOWN";
}

const char* mhc_last_error_message(void) { return g_msg; }

// ---- expansion rate 4 (the page's operation) ------------------------------

mhc_status mhc_h_aggregate_validate_fwd(const uint16_t* residual, const float* pre,
                                        const uint16_t* out, int64_t T, int64_t H) {
  return validate_fwd(residual, pre, out, T, MHC_HC, H);
}

mhc_status mhc_h_aggregate_validate_bwd(const uint16_t* residual, const float* pre,
                                        const uint16_t* grad_out,
                                        const uint16_t* grad_residual, const float* grad_pre,
                                        int64_t T, int64_t H) {
  return validate_bwd(residual, pre, grad_out, grad_residual, grad_pre, T, MHC_HC, H);
}

mhc_status mhc_h_aggregate_plan_fwd(const uint16_t* residual, const float* pre,
                                    const uint16_t* out, int64_t T, int64_t H,
                                    const mhc_launch* launch, mhc_launch* plan,
                                    int64_t* grid_blocks) {
  return plan_fwd_query(residual, pre, out, T, MHC_HC, H, launch, plan, grid_blocks);
}

mhc_status mhc_h_aggregate_plan_bwd(const uint16_t* residual, const float* pre,
                                    const uint16_t* grad_out, const uint16_t* grad_residual,
                                    const float* grad_pre, int64_t T, int64_t H,
                                    const mhc_launch* launch, mhc_launch* plan,
                                    int64_t* grid_blocks) {
  return plan_bwd_query(residual, pre, grad_out, grad_residual, grad_pre, T, MHC_HC, H, false,
                        launch, plan, grid_blocks);
}

mhc_status mhc_h_aggregate_plan_bwd_acc(const uint16_t* residual, const float* pre,
                                        const uint16_t* grad_out, const uint16_t* grad_residual,
                                        const float* grad_pre, int64_t T, int64_t H,
                                        const mhc_launch* launch, mhc_launch* plan,
                                        int64_t* grid_blocks) {
  return plan_bwd_query(residual, pre, grad_out, grad_residual, grad_pre, T, MHC_HC, H, true,
                        launch, plan, grid_blocks);
}

mhc_status mhc_h_aggregate_fwd(const uint16_t* residual, const float* pre, uint16_t* out,
                               int64_t T, int64_t H, void* stream) {
  return run_fwd(residual, pre, out, T, MHC_HC, H, stream, nullptr, events(nullptr, nullptr));
}

mhc_status mhc_h_aggregate_fwd_ex(const uint16_t* residual, const float* pre, uint16_t* out,
                                  int64_t T, int64_t H, void* stream,
                                  const mhc_launch* launch) {
  return run_fwd(residual, pre, out, T, MHC_HC, H, stream, launch, events(nullptr, nullptr));
}

mhc_status mhc_h_aggregate_fwd_timed(const uint16_t* residual, const float* pre, uint16_t* out,
                                     int64_t T, int64_t H, void* stream,
                                     const mhc_launch* launch, void* start_event,
                                     void* stop_event) {
  return run_fwd(residual, pre, out, T, MHC_HC, H, stream, launch,
                 events(start_event, stop_event));
}

mhc_status mhc_h_aggregate_bwd(const uint16_t* residual, const float* pre,
                               const uint16_t* grad_out, uint16_t* grad_residual,
                               float* grad_pre, int64_t T, int64_t H, void* stream) {
  return run_bwd(residual, pre, grad_out, grad_residual, grad_pre, T, MHC_HC, H, false, stream,
                 nullptr, events(nullptr, nullptr));
}

mhc_status mhc_h_aggregate_bwd_ex(const uint16_t* residual, const float* pre,
                                  const uint16_t* grad_out, uint16_t* grad_residual,
                                  float* grad_pre, int64_t T, int64_t H, void* stream,
                                  const mhc_launch* launch) {
  return run_bwd(residual, pre, grad_out, grad_residual, grad_pre, T, MHC_HC, H, false, stream,
                 launch, events(nullptr, nullptr));
}

mhc_status mhc_h_aggregate_bwd_timed(const uint16_t* residual, const float* pre,
                                     const uint16_t* grad_out, uint16_t* grad_residual,
                                     float* grad_pre, int64_t T, int64_t H, void* stream,
                                     const mhc_launch* launch, void* start_event,
                                     void* stop_event) {
  return run_bwd(residual, pre, grad_out, grad_residual, grad_pre, T, MHC_HC, H, false, stream,
                 launch, events(start_event, stop_event));
}

mhc_status mhc_h_aggregate_bwd_acc(const uint16_t* residual, const float* pre,
                                   const uint16_t* grad_out, uint16_t* grad_residual,
                                   float* grad_pre, int64_t T, int64_t H, void* stream,
                                   const mhc_launch* launch, void* start_event,
                                   void* stop_event) {
  return run_bwd(residual, pre, grad_out, grad_residual, grad_pre, T, MHC_HC, H, true, stream,
                 launch, events(start_event, stop_event));
}

// ---- any supported expansion rate -----------------------------------------

mhc_status mhc_h_aggregate_fwd_n(const uint16_t* residual, const float* pre, uint16_t* out,
                                 int64_t T, int32_t n, int64_t H, void* stream,
                                 const mhc_launch* launch, void* start_event, void* stop_event) {
  return run_fwd(residual, pre, out, T, n, H, stream, launch, events(start_event, stop_event));
}

mhc_status mhc_h_aggregate_bwd_n(const uint16_t* residual, const float* pre,
                                 const uint16_t* grad_out, uint16_t* grad_residual,
                                 float* grad_pre, int64_t T, int32_t n, int64_t H,
                                 int32_t accumulate, void* stream, const mhc_launch* launch,
                                 void* start_event, void* stop_event) {
  if (accumulate != 0 && accumulate != 1)
    return fail(MHC_ERROR_INVALID_VALUE, "accumulate must be 0 or 1");
  return run_bwd(residual, pre, grad_out, grad_residual, grad_pre, T, n, H, accumulate == 1,
                 stream, launch, events(start_event, stop_event));
}

mhc_status mhc_h_aggregate_plan_fwd_n(const uint16_t* residual, const float* pre,
                                      const uint16_t* out, int64_t T, int32_t n, int64_t H,
                                      const mhc_launch* launch, mhc_launch* plan,
                                      int64_t* grid_blocks) {
  return plan_fwd_query(residual, pre, out, T, n, H, launch, plan, grid_blocks);
}

mhc_status mhc_h_aggregate_plan_bwd_n(const uint16_t* residual, const float* pre,
                                      const uint16_t* grad_out, const uint16_t* grad_residual,
                                      const float* grad_pre, int64_t T, int32_t n, int64_t H,
                                      int32_t accumulate, const mhc_launch* launch,
                                      mhc_launch* plan, int64_t* grid_blocks) {
  if (accumulate != 0 && accumulate != 1)
    return fail(MHC_ERROR_INVALID_VALUE, "accumulate must be 0 or 1");
  return plan_bwd_query(residual, pre, grad_out, grad_residual, grad_pre, T, n, H,
                        accumulate == 1, launch, plan, grid_blocks);
}

}  // extern "C"
