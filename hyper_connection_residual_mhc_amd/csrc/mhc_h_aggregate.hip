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
//  * Backward: one block of 4 waves (256 lanes) owns a token; each lane
//    streams its 8-element groups in the fixed lane order, writes
//    grad_residual on the way and keeps 4 fp32 accumulators, which a
//    fixed-order cross-lane tree and an LDS step reduce to grad_pre[t,:].
//  * Bit exactness: contraction is off for the whole file (pragma and
//    -ffp-contract=off), fast-math builds are refused, fp32 denormals are
//    kept (the kernel descriptor's default mode), and every bf16 result goes
//    through the hardware round-to-nearest-even pack conversion.

#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "mhc_h_aggregate.h"

#if defined(__FAST_MATH__)
#error "mhc_h_aggregate must not be built with fast-math: its results are defined bit for bit"
#endif

#pragma clang fp contract(off)

namespace {

// ---------------------------------------------------------------------------
// Device helpers: exact widening and round-to-nearest-even narrowing
// ---------------------------------------------------------------------------

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 values -> two bf16 patterns packed low|high in one dword, rounded
// to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ uint16_t to_bf16(float x) {
  return static_cast<uint16_t>(pack_bf16x2(x, 0.0f));
}

// bf16 pattern -> fp32, exact (the bf16 pattern is the top half of the fp32).
__device__ __forceinline__ float lo_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// A V-element bf16 vector as the widest plain integer type of that size.
template <int V> struct Vec;
template <> struct Vec<8> { typedef uint4 type; };
template <> struct Vec<4> { typedef uint2 type; };
template <> struct Vec<2> { typedef uint32_t type; };
template <> struct Vec<1> { typedef uint16_t type; };

// Element e of a vector, widened to fp32.
template <int V>
__device__ __forceinline__ float elem(const typename Vec<V>::type& v, int e);
template <> __device__ __forceinline__ float elem<8>(const uint4& v, int e) {
  const uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
  return (e & 1) ? hi_f32(w) : lo_f32(w);
}
template <> __device__ __forceinline__ float elem<4>(const uint2& v, int e) {
  const uint32_t w = e < 2 ? v.x : v.y;
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
template <> __device__ __forceinline__ uint4 pack<8>(const float (&y)[8]) {
  return make_uint4(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]),
                    pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7]));
}
template <> __device__ __forceinline__ uint2 pack<4>(const float (&y)[4]) {
  return make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
}
template <> __device__ __forceinline__ uint32_t pack<2>(const float (&y)[2]) {
  return pack_bf16x2(y[0], y[1]);
}
template <> __device__ __forceinline__ uint16_t pack<1>(const float (&y)[1]) {
  return to_bf16(y[0]);
}

template <int V>
__device__ __forceinline__ typename Vec<V>::type load_vec(const uint16_t* p) {
  return *reinterpret_cast<const typename Vec<V>::type*>(p);
}
template <int V>
__device__ __forceinline__ void store_vec(uint16_t* p, const typename Vec<V>::type& v) {
  *reinterpret_cast<typename Vec<V>::type*>(p) = v;
}

// ---------------------------------------------------------------------------
// Forward kernel
// ---------------------------------------------------------------------------
//
// Grid: blocks_per_token * T blocks of blockDim.x threads (a multiple of 64).
// Block b serves token t = b / blocks_per_token and, within it, the units
// [c * blockDim.x * UPT, (c + 1) * blockDim.x * UPT) with c = b mod
// blocks_per_token; a unit is V consecutive hidden elements. Lane x of the
// block owns units c*blockDim.x*UPT + k*blockDim.x + x for k < UPT, so every
// load and store instruction of a wave covers 64 consecutive units.
// All loads of a lane are issued before any arithmetic.
template <int V, int UPT>
__global__ __launch_bounds__(1024) void hagg_fwd_kernel(
    const uint16_t* __restrict__ residual, const float* __restrict__ pre,
    uint16_t* __restrict__ out, int64_t H, uint32_t units_per_token,
    uint32_t blocks_per_token) {
  typedef typename Vec<V>::type VT;
  const uint32_t b = blockIdx.x;
  const uint32_t t = b / blocks_per_token;
  const uint32_t c = b - t * blocks_per_token;

  const float* p = pre + 4 * static_cast<int64_t>(t);
  const float w0 = p[0], w1 = p[1], w2 = p[2], w3 = p[3];
  const uint16_t* r0 = residual + static_cast<int64_t>(t) * 4 * H;
  const uint16_t* r1 = r0 + H;
  const uint16_t* r2 = r1 + H;
  const uint16_t* r3 = r2 + H;
  uint16_t* o = out + static_cast<int64_t>(t) * H;

  const uint32_t first = c * blockDim.x * UPT + threadIdx.x;

  VT x0[UPT], x1[UPT], x2[UPT], x3[UPT];
#pragma unroll
  for (int k = 0; k < UPT; ++k) {
    const uint32_t u = first + k * blockDim.x;
    if (u < units_per_token) {
      const int64_t h = static_cast<int64_t>(u) * V;
      x0[k] = load_vec<V>(r0 + h);
      x1[k] = load_vec<V>(r1 + h);
      x2[k] = load_vec<V>(r2 + h);
      x3[k] = load_vec<V>(r3 + h);
    }
  }
#pragma unroll
  for (int k = 0; k < UPT; ++k) {
    const uint32_t u = first + k * blockDim.x;
    if (u < units_per_token) {
      float y[V];
#pragma unroll
      for (int e = 0; e < V; ++e) {
        // Separate fp32 round-to-nearest products and sums, tree (0+1)+(2+3).
        const float p0 = w0 * elem<V>(x0[k], e);
        const float p1 = w1 * elem<V>(x1[k], e);
        const float p2 = w2 * elem<V>(x2[k], e);
        const float p3 = w3 * elem<V>(x3[k], e);
        const float s01 = p0 + p1;
        const float s23 = p2 + p3;
        y[e] = s01 + s23;
      }
      store_vec<V>(o + static_cast<int64_t>(u) * V, pack<V>(y));
    }
  }
}

// ---------------------------------------------------------------------------
// Backward kernel
// ---------------------------------------------------------------------------
//
// Grid: ceil(T / tokens_per_block) blocks of exactly 256 threads. Lane l
// (= threadIdx.x) is accumulator lane l of the fixed order: it visits groups
// k = l, l + 256, l + 512, ... (group k = hidden elements 8k .. 8k+7), U of
// them per batch of loads, and for each element adds grad_out*residual_i to
// its accumulator i in ascending h. It also writes grad_residual for every
// element it visits. Then each wave halves its 64 accumulators with
// offsets 32..1 and the four wave results meet in LDS as (y0+y2)+(y1+y3).
// V elements are moved per access; V divides 8 and H, so a group is 8/V
// accesses (fewer for a short last group).
constexpr int kGroup = 8;
constexpr int kLanes = 256;

template <int V, int U>
__global__ __launch_bounds__(256) void hagg_bwd_kernel(
    const uint16_t* __restrict__ residual, const float* __restrict__ pre,
    const uint16_t* __restrict__ grad_out, uint16_t* __restrict__ grad_residual,
    float* __restrict__ grad_pre, int64_t T, int64_t H, int64_t ngroups,
    int32_t tokens_per_block) {
  typedef typename Vec<V>::type VT;
  constexpr int NV = kGroup / V;  // accesses per full group
  __shared__ float wave_sum[4][4];  // [wave][stream]

  const int lane = threadIdx.x;
  const int wave = lane >> 6;

  for (int32_t tt = 0; tt < tokens_per_block; ++tt) {
    const int64_t t = static_cast<int64_t>(blockIdx.x) * tokens_per_block + tt;
    if (t >= T) break;  // uniform across the block

    const float* p = pre + 4 * t;
    const float w[4] = {p[0], p[1], p[2], p[3]};
    const uint16_t* g_row = grad_out + t * H;
    const uint16_t* r_row = residual + t * 4 * H;
    uint16_t* gr_row = grad_residual + t * 4 * H;

    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};

    for (int64_t k0 = lane; k0 < ngroups; k0 += static_cast<int64_t>(kLanes) * U) {
      VT g[U][NV];
      VT r[U][NV][4];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t k = k0 + static_cast<int64_t>(u) * kLanes;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          const int64_t h = k * kGroup + v * V;
          if (k < ngroups && h < H) {
            g[u][v] = load_vec<V>(g_row + h);
#pragma unroll
            for (int i = 0; i < 4; ++i) r[u][v][i] = load_vec<V>(r_row + i * H + h);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t k = k0 + static_cast<int64_t>(u) * kLanes;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          const int64_t h = k * kGroup + v * V;
          if (k < ngroups && h < H) {
            float gr[4][V];
#pragma unroll
            for (int e = 0; e < V; ++e) {
              const float ge = elem<V>(g[u][v], e);
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                gr[i][e] = w[i] * ge;
                const float q = ge * elem<V>(r[u][v][i], e);  // exact in the normal range
                acc[i] = acc[i] + q;
              }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) store_vec<V>(gr_row + i * H + h, pack<V>(gr[i]));
          }
        }
      }
    }

    // Wave stage: x[j] = x[j] + x[j + off] for off = 32, 16, 8, 4, 2, 1.
    // Lanes j >= off compute values nobody reads.
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = acc[i] + __shfl_down(acc[i], off, 64);
    }
    if ((lane & 63) == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) wave_sum[wave][i] = acc[i];
    }
    __syncthreads();
    if (lane < 4) {
      const float y02 = wave_sum[0][lane] + wave_sum[2][lane];
      const float y13 = wave_sum[1][lane] + wave_sum[3][lane];
      grad_pre[4 * t + lane] = y02 + y13;
    }
    __syncthreads();  // wave_sum is reused by the next token
  }
}

// ---------------------------------------------------------------------------
// Conversion probe kernel
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bf16_probe_kernel(uint32_t first_bits,
                                                         int64_t n,
                                                         uint16_t* __restrict__ out) {
  const int64_t k = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (k >= n) return;
  const uint32_t bits = first_bits + static_cast<uint32_t>(k);
  out[k] = to_bf16(__uint_as_float(bits));
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

// Byte sizes of every tensor, or an error if T, H or the sizes are invalid.
struct Sizes {
  int64_t res_bytes, pre_bytes, row_bytes;  // row = [T,H] bf16
};

mhc_status check_sizes(int64_t T, int64_t H, Sizes* s) {
  if (T < 0) return fail(MHC_ERROR_INVALID_VALUE, "T must be >= 0 (got %lld)", (long long)T);
  if (H < 1 || H > MHC_MAX_H)
    return fail(MHC_ERROR_INVALID_VALUE, "H must be in [1, %lld] (got %lld)",
                (long long)MHC_MAX_H, (long long)H);
  // 8*T*H must fit int64 (residual bytes).
  if (T > INT64_MAX / 8 / H)
    return fail(MHC_ERROR_INVALID_VALUE, "T*H too large: byte counts overflow int64");
  s->res_bytes = 8 * T * H;
  s->row_bytes = 2 * T * H;
  s->pre_bytes = 16 * T;
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

// MI355X: 256 compute units (8 XCDs x 32).
constexpr int64_t kTargetCUs = 256;
// One dispatch covers at most 2^31 work-items (the AQL packet's grid size is a
// 32-bit work-item count); larger problems are split over whole tokens.
constexpr int64_t kMaxLaunchThreads = int64_t(1) << 31;

struct FwdPlan {
  int V, block, upt;
  uint32_t units_per_token, blocks_per_token;
  int64_t tokens_per_launch, total_blocks;
};

mhc_status plan_fwd(const uint16_t* residual, const uint16_t* out, int64_t T, int64_t H,
                    const mhc_launch* ov, FwdPlan* pl) {
  const void* bufs[2] = {residual, out};
  int V = widest_vec(H, bufs, 2);
  if (ov && ov->vec_width != 0) {
    if (!vec_allowed(ov->vec_width, H, bufs, 2))
      return fail(MHC_ERROR_INVALID_VALUE,
                  "vec_width %d not allowed for H=%lld and the buffers' alignment",
                  ov->vec_width, (long long)H);
    V = ov->vec_width;
  }
  const int64_t upt_units = H / V;  // units per token
  int upt = 1;
  if (ov && ov->units_per_thread != 0) {
    if (ov->units_per_thread != 1 && ov->units_per_thread != 2 && ov->units_per_thread != 4)
      return fail(MHC_ERROR_INVALID_VALUE, "units_per_thread must be 1, 2 or 4");
    upt = ov->units_per_thread;
  }
  int block;
  if (ov && ov->block_threads != 0) {
    if (ov->block_threads < 64 || ov->block_threads > 1024 || ov->block_threads % 64 != 0)
      return fail(MHC_ERROR_INVALID_VALUE, "block_threads must be a multiple of 64 in [64, 1024]");
    block = ov->block_threads;
  } else if (T * upt_units < kTargetCUs * 256) {
    // Fewer units than one 256-thread block per CU: small blocks spread the
    // few units over as many CUs as possible (latency-bound regime).
    block = 64;
  } else {
    // Bandwidth regime: the larger of 256 / 128 that leaves the fewest idle
    // lanes in a token's last block.
    const int64_t span256 = 256LL * upt, span128 = 128LL * upt;
    const int64_t idle256 = ((upt_units + span256 - 1) / span256) * span256 - upt_units;
    const int64_t idle128 = ((upt_units + span128 - 1) / span128) * span128 - upt_units;
    block = idle128 < idle256 ? 128 : 256;
  }
  const int64_t span = static_cast<int64_t>(block) * upt;
  const int64_t bpt = (upt_units + span - 1) / span;
  pl->V = V;
  pl->block = block;
  pl->upt = upt;
  pl->units_per_token = static_cast<uint32_t>(upt_units);
  pl->blocks_per_token = static_cast<uint32_t>(bpt);
  int64_t tpl = kMaxLaunchThreads / (bpt * block);
  if (tpl < 1) tpl = 1;  // cannot happen for H <= MHC_MAX_H
  pl->tokens_per_launch = tpl;
  pl->total_blocks = T * bpt;
  return ok();
}

struct BwdPlan {
  int V, U, tpb;
  int64_t ngroups, blocks_per_launch, total_blocks;
};

mhc_status plan_bwd(const uint16_t* residual, const uint16_t* grad_out,
                    const uint16_t* grad_residual, int64_t T, int64_t H,
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
  if (ov && ov->block_threads != 0 && ov->block_threads != kLanes)
    return fail(MHC_ERROR_INVALID_VALUE, "backward block_threads must be 0 or 256");
  // Groups each lane loads before its arithmetic: two 16-byte groups (160
  // bytes of input) keep the kernel near 80 VGPRs, so all blocks of a
  // 1024-token call are resident at once; narrower accesses already issue
  // many loads per group.
  int U = V == 8 ? 2 : 1;
  if (ov && ov->units_per_thread != 0) {
    if (ov->units_per_thread != 1 && ov->units_per_thread != 2 && ov->units_per_thread != 4)
      return fail(MHC_ERROR_INVALID_VALUE, "units_per_thread must be 1, 2 or 4");
    U = ov->units_per_thread;
  }
  int tpb = 1;
  if (ov && ov->tokens_per_block != 0) {
    if (ov->tokens_per_block < 1 || ov->tokens_per_block > 4096)
      return fail(MHC_ERROR_INVALID_VALUE, "tokens_per_block must be in [1, 4096]");
    tpb = ov->tokens_per_block;
  }
  pl->V = V;
  pl->U = U;
  pl->tpb = tpb;
  pl->ngroups = (H + kGroup - 1) / kGroup;
  pl->blocks_per_launch = kMaxLaunchThreads / kLanes;
  pl->total_blocks = (T + tpb - 1) / tpb;
  return ok();
}

mhc_status validate_fwd(const uint16_t* residual, const float* pre, const uint16_t* out,
                        int64_t T, int64_t H) {
  Sizes s;
  mhc_status st = check_sizes(T, H, &s);
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
                        int64_t H) {
  Sizes s;
  mhc_status st = check_sizes(T, H, &s);
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

mhc_status launch_error(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(MHC_ERROR_HIP, "%s launch failed: %s (%s)", what, hipGetErrorName(e),
                hipGetErrorString(e));
  return ok();
}

template <int V, int UPT>
void launch_fwd_t(const FwdPlan& pl, const uint16_t* residual, const float* pre, uint16_t* out,
                  int64_t tokens, int64_t H, hipStream_t stream) {
  const uint32_t blocks = static_cast<uint32_t>(tokens * pl.blocks_per_token);
  hagg_fwd_kernel<V, UPT><<<dim3(blocks), dim3(pl.block), 0, stream>>>(
      residual, pre, out, H, pl.units_per_token, pl.blocks_per_token);
}

template <int V>
void launch_fwd_v(const FwdPlan& pl, const uint16_t* residual, const float* pre, uint16_t* out,
                  int64_t tokens, int64_t H, hipStream_t stream) {
  switch (pl.upt) {
    case 1: launch_fwd_t<V, 1>(pl, residual, pre, out, tokens, H, stream); break;
    case 2: launch_fwd_t<V, 2>(pl, residual, pre, out, tokens, H, stream); break;
    default: launch_fwd_t<V, 4>(pl, residual, pre, out, tokens, H, stream); break;
  }
}

template <int V, int U>
void launch_bwd_t(const BwdPlan& pl, const uint16_t* residual, const float* pre,
                  const uint16_t* grad_out, uint16_t* grad_residual, float* grad_pre,
                  int64_t tokens, int64_t H, hipStream_t stream) {
  const uint32_t blocks = static_cast<uint32_t>((tokens + pl.tpb - 1) / pl.tpb);
  hagg_bwd_kernel<V, U><<<dim3(blocks), dim3(kLanes), 0, stream>>>(
      residual, pre, grad_out, grad_residual, grad_pre, tokens, H, pl.ngroups, pl.tpb);
}

template <int V>
void launch_bwd_v(const BwdPlan& pl, const uint16_t* residual, const float* pre,
                  const uint16_t* grad_out, uint16_t* grad_residual, float* grad_pre,
                  int64_t tokens, int64_t H, hipStream_t stream) {
  switch (pl.U) {
    case 1: launch_bwd_t<V, 1>(pl, residual, pre, grad_out, grad_residual, grad_pre, tokens, H, stream); break;
    case 2: launch_bwd_t<V, 2>(pl, residual, pre, grad_out, grad_residual, grad_pre, tokens, H, stream); break;
    default: launch_bwd_t<V, 4>(pl, residual, pre, grad_out, grad_residual, grad_pre, tokens, H, stream); break;
  }
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

mhc_status mhc_h_aggregate_validate_fwd(const uint16_t* residual, const float* pre,
                                        const uint16_t* out, int64_t T, int64_t H) {
  return validate_fwd(residual, pre, out, T, H);
}

mhc_status mhc_h_aggregate_validate_bwd(const uint16_t* residual, const float* pre,
                                        const uint16_t* grad_out,
                                        const uint16_t* grad_residual, const float* grad_pre,
                                        int64_t T, int64_t H) {
  return validate_bwd(residual, pre, grad_out, grad_residual, grad_pre, T, H);
}

mhc_status mhc_h_aggregate_plan_fwd(const uint16_t* residual, const float* pre,
                                    const uint16_t* out, int64_t T, int64_t H,
                                    const mhc_launch* launch, mhc_launch* plan,
                                    int64_t* grid_blocks) {
  mhc_status st = validate_fwd(residual, pre, out, T, H);
  if (st != MHC_SUCCESS) return st;
  FwdPlan pl;
  if ((st = plan_fwd(residual, out, T, H, launch, &pl)) != MHC_SUCCESS) return st;
  if (plan) *plan = mhc_launch{pl.block, pl.V, pl.upt, 0};
  if (grid_blocks) *grid_blocks = pl.total_blocks;
  return ok();
}

mhc_status mhc_h_aggregate_plan_bwd(const uint16_t* residual, const float* pre,
                                    const uint16_t* grad_out, const uint16_t* grad_residual,
                                    const float* grad_pre, int64_t T, int64_t H,
                                    const mhc_launch* launch, mhc_launch* plan,
                                    int64_t* grid_blocks) {
  mhc_status st = validate_bwd(residual, pre, grad_out, grad_residual, grad_pre, T, H);
  if (st != MHC_SUCCESS) return st;
  BwdPlan pl;
  if ((st = plan_bwd(residual, grad_out, grad_residual, T, H, launch, &pl)) != MHC_SUCCESS)
    return st;
  if (plan) *plan = mhc_launch{kLanes, pl.V, pl.U, pl.tpb};
  if (grid_blocks) *grid_blocks = pl.total_blocks;
  return ok();
}

mhc_status mhc_h_aggregate_fwd_ex(const uint16_t* residual, const float* pre, uint16_t* out,
                                  int64_t T, int64_t H, void* stream,
                                  const mhc_launch* launch) {
  mhc_status st = validate_fwd(residual, pre, out, T, H);
  if (st != MHC_SUCCESS || T == 0) return st;
  FwdPlan pl;
  if ((st = plan_fwd(residual, out, T, H, launch, &pl)) != MHC_SUCCESS) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // start from a clean per-thread error state
  for (int64_t t0 = 0; t0 < T; t0 += pl.tokens_per_launch) {
    const int64_t n = (T - t0 < pl.tokens_per_launch) ? T - t0 : pl.tokens_per_launch;
    const uint16_t* r = residual + t0 * 4 * H;
    const float* p = pre + 4 * t0;
    uint16_t* o = out + t0 * H;
    switch (pl.V) {
      case 8: launch_fwd_v<8>(pl, r, p, o, n, H, s); break;
      case 4: launch_fwd_v<4>(pl, r, p, o, n, H, s); break;
      case 2: launch_fwd_v<2>(pl, r, p, o, n, H, s); break;
      default: launch_fwd_v<1>(pl, r, p, o, n, H, s); break;
    }
    if ((st = launch_error("h_aggregate forward")) != MHC_SUCCESS) return st;
  }
  return ok();
}

mhc_status mhc_h_aggregate_fwd(const uint16_t* residual, const float* pre, uint16_t* out,
                               int64_t T, int64_t H, void* stream) {
  return mhc_h_aggregate_fwd_ex(residual, pre, out, T, H, stream, nullptr);
}

mhc_status mhc_h_aggregate_bwd_ex(const uint16_t* residual, const float* pre,
                                  const uint16_t* grad_out, uint16_t* grad_residual,
                                  float* grad_pre, int64_t T, int64_t H, void* stream,
                                  const mhc_launch* launch) {
  mhc_status st = validate_bwd(residual, pre, grad_out, grad_residual, grad_pre, T, H);
  if (st != MHC_SUCCESS || T == 0) return st;
  BwdPlan pl;
  if ((st = plan_bwd(residual, grad_out, grad_residual, T, H, launch, &pl)) != MHC_SUCCESS)
    return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t tokens_per_launch = pl.blocks_per_launch * pl.tpb;
  (void)hipGetLastError();
  for (int64_t t0 = 0; t0 < T; t0 += tokens_per_launch) {
    const int64_t n = (T - t0 < tokens_per_launch) ? T - t0 : tokens_per_launch;
    const uint16_t* r = residual + t0 * 4 * H;
    const float* p = pre + 4 * t0;
    const uint16_t* g = grad_out + t0 * H;
    uint16_t* gr = grad_residual + t0 * 4 * H;
    float* gp = grad_pre + 4 * t0;
    switch (pl.V) {
      case 8: launch_bwd_v<8>(pl, r, p, g, gr, gp, n, H, s); break;
      case 4: launch_bwd_v<4>(pl, r, p, g, gr, gp, n, H, s); break;
      case 2: launch_bwd_v<2>(pl, r, p, g, gr, gp, n, H, s); break;
      default: launch_bwd_v<1>(pl, r, p, g, gr, gp, n, H, s); break;
    }
    if ((st = launch_error("h_aggregate backward")) != MHC_SUCCESS) return st;
  }
  return ok();
}

mhc_status mhc_h_aggregate_bwd(const uint16_t* residual, const float* pre,
                               const uint16_t* grad_out, uint16_t* grad_residual,
                               float* grad_pre, int64_t T, int64_t H, void* stream) {
  return mhc_h_aggregate_bwd_ex(residual, pre, grad_out, grad_residual, grad_pre, T, H, stream,
                                nullptr);
}

mhc_status mhc_bf16_rne_probe(uint32_t first_bits, int64_t n, uint16_t* out, void* stream) {
  if (n < 0 || n > (int64_t(1) << 32))
    return fail(MHC_ERROR_INVALID_VALUE, "n must be in [0, 2^32]");
  if (n == 0) return ok();
  mhc_status st = check_ptr(out, 2, "out");
  if (st != MHC_SUCCESS) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const int64_t per_launch = int64_t(1) << 30;  // work-items per dispatch
  for (int64_t k0 = 0; k0 < n; k0 += per_launch) {
    const int64_t m = (n - k0 < per_launch) ? n - k0 : per_launch;
    const uint32_t blocks = static_cast<uint32_t>((m + 255) / 256);
    bf16_probe_kernel<<<dim3(blocks), dim3(256), 0, s>>>(
        first_bits + static_cast<uint32_t>(k0), m, out + k0);
    if ((st = launch_error("bf16 probe")) != MHC_SUCCESS) return st;
  }
  return ok();
}

}  // extern "C"
