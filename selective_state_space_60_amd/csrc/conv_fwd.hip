// Causal depthwise convolution (+ bias, + SiLU) for gfx950: the Mamba block's
// per-channel Conv1D of width W in front of the scan ("Mamba 논문 리뷰",
// tildalice.io, Mamba 블록 아키텍처 and the SelectiveSSM listing: W - 1 steps of
// zero padding, output cut back to the first L steps, then SiLU):
//   y[b,t,d] = silu(bias[d] + sum_k w[d,k] x[b, t-W+1+k, d]),  x = 0 for t < 0.
// Bound by HBM: every x is read once and every y written once.  A thread owns
// V consecutive channels (4 with aligned rows, else 1) and a run of TS time
// steps; it loads the run and the W - 1 steps before it with one load per
// step issued up front, keeps them in registers and slides the window there.
// A wave covers 64 * V consecutive channels, so every load and store of a
// step is one contiguous row segment.  The left padding of the first run and
// the rows past the sequence come back as zeros from the buffer range check,
// so no load sits behind a branch.
#include <hip/hip_runtime.h>

#include "ssm_internal.h"

namespace ssm {
namespace {

constexpr int NT = 256;
constexpr int TS = 32;  // time steps per thread
static_assert(TS >= kConvMaxWidth - 1, "a run's padding rows must all precede it");
constexpr float kLog2e = 1.4426950408889634f;

constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw (unformatted) buffer access
constexpr uint32_t kFar = 0x40000000u;        // an offset past every range: reads return 0

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t range) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)range, (int)kRsrcWord3);
}

template <bool BF16, int V>
struct Row {
  uint32_t w[BF16 ? (V + 1) / 2 : V];
};

template <bool BF16, int V>
__device__ __forceinline__ Row<BF16, V> load_row(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  Row<BF16, V> o;
  if constexpr (BF16 && V == 4) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
    o.w[0] = v[0]; o.w[1] = v[1];
  } else if constexpr (!BF16 && V == 4) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    o.w[0] = v[0]; o.w[1] = v[1]; o.w[2] = v[2]; o.w[3] = v[3];
  } else if constexpr (BF16) {
    o.w[0] = __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
  } else {
    o.w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
  }
  return o;
}

template <bool BF16, int V>
__device__ __forceinline__ float elem(const Row<BF16, V>& r, int v) {
  if constexpr (BF16) {
    if constexpr (V == 1) return __uint_as_float(r.w[0] << 16);
    else return __uint_as_float((v & 1) ? (r.w[v >> 1] & 0xFFFF0000u) : (r.w[v >> 1] << 16));
  } else {
    return __uint_as_float(r.w[v]);
  }
}

// Two floats to a bf16 pair (a in the low half), round to nearest even: one
// v_cvt_pk_bf16_f32 (converting each float alone and merging the halves
// takes four instructions).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

template <bool BF16, bool YF32, int V>
__device__ __forceinline__ void store_row(__amdgpu_buffer_rsrc_t r, uint32_t off, const float (&o)[V]) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  if constexpr (YF32 || !BF16) {
    if constexpr (V == 4) {
      const u32x4 w = {__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]), __float_as_uint(o[3])};
      __builtin_amdgcn_raw_buffer_store_b128(w, r, (int)off, 0, 0);
    } else {
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o[0]), r, (int)off, 0, 0);
    }
  } else {
    if constexpr (V == 4) {
      u32x2 w;
      w[0] = pack2(o[0], o[1]);
      w[1] = pack2(o[2], o[3]);
      __builtin_amdgcn_raw_buffer_store_b64(w, r, (int)off, 0, 0);
    } else {
      __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (__bf16)o[0]), r, (int)off, 0, 0);
    }
  }
}

// Every access is a buffer access relative to the first channel of the
// workgroup in the run's first row, so an address is the lane's fixed byte
// offset plus a multiple of the row stride (32-bit, checked on the host).
template <bool BF16, bool YF32, int V, int W, bool SILU>
__global__ __launch_bounds__(NT) void conv_kernel(ConvParams p, unsigned nchb, unsigned ntc) {
  constexpr int E = BF16 ? 2 : 4;
  constexpr int YE = (YF32 || !BF16) ? 4 : 2;
  const unsigned blk = blockIdx.x;
  const unsigned cg = blk % nchb;
  const unsigned tc = (blk / nchb) % ntc;
  const int64_t b = blk / (nchb * ntc);
  const int64_t c0 = (int64_t)cg * NT * V;  // first channel of the workgroup
  const int64_t d0 = c0 + (int64_t)threadIdx.x * V;
  if (d0 >= p.D) return;  // V divides D on the vector path, so a thread is all in or all out
  const int64_t t0 = (int64_t)tc * TS;
  // first row read: W - 1 steps before the run, or step 0 for the first run,
  // whose W - 1 steps of left padding read at kFar (zeros)
  const int64_t tb = t0 > 0 ? t0 - (W - 1) : 0;
  const int skip = t0 > 0 ? 0 : W - 1;

  float wv[V][W], bv[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
#pragma unroll
    for (int k = 0; k < W; ++k) wv[v][k] = p.w[(d0 + v) * p.ws_d + k * p.ws_k];
    bv[v] = p.bias ? p.bias[(d0 + v) * p.bs_d] : 0.f;
  }
  // x: range ends after the last channel of row L-1 (rows past the sequence
  // read zeros), capped below kFar
  const int64_t xr = ((p.L - 1 - tb) * p.xs_t + (p.D - c0)) * E;
  const __amdgpu_buffer_rsrc_t rx =
      rsrc((const char*)p.x + (b * p.xs_b + tb * p.xs_t + c0) * E, (uint32_t)(xr < (int64_t)kFar ? xr : kFar - 1));
  const uint32_t lane_x = (uint32_t)(threadIdx.x * V * E);
  const uint32_t row_x = (uint32_t)(p.xs_t * E);
  constexpr int R = TS + W - 1;
  Row<BF16, V> rows[R];
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const uint32_t off = j < skip ? kFar : lane_x + (uint32_t)(j - skip) * row_x;
    rows[j] = load_row<BF16, V>(rx, off);
  }
  // y: range ends after the last channel of row L-1, so the stores of steps
  // past the sequence are dropped (the host passes a row stride >= D)
  const int64_t yr = ((p.L - 1 - t0) * p.ys_t + (p.D - c0)) * YE;
  const __amdgpu_buffer_rsrc_t ry =
      rsrc((char*)p.y + (b * p.ys_b + t0 * p.ys_t + c0) * YE, (uint32_t)(yr < (int64_t)kFar ? yr : kFar - 1));
  const uint32_t lane_y = (uint32_t)(threadIdx.x * V * YE);
  const uint32_t row_y = (uint32_t)(p.ys_t * YE);
#pragma unroll
  for (int j = 0; j < TS; ++j) {
    float o[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      float acc = bv[v];
#pragma unroll
      for (int k = 0; k < W; ++k) acc = __builtin_fmaf(wv[v][k], elem<BF16, V>(rows[j + k], v), acc);
      if constexpr (SILU) acc *= __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-acc * kLog2e));
      o[v] = acc;
    }
    store_row<BF16, YF32, V>(ry, lane_y + (uint32_t)j * row_y, o);
  }
}

template <bool BF16, int V, int W>
void launch_w(const ConvParams& p, hipStream_t stream) {
  const unsigned nchb = (unsigned)((p.D + (int64_t)NT * V - 1) / ((int64_t)NT * V));
  const unsigned ntc = (unsigned)((p.L + TS - 1) / TS);
  const dim3 grid(nchb * ntc * (unsigned)p.batch);
  const bool yf = p.y_f32 || !BF16;
  if (p.silu) {
    if (yf) hipLaunchKernelGGL((conv_kernel<BF16, true, V, W, true>), grid, dim3(NT), 0, stream, p, nchb, ntc);
    else hipLaunchKernelGGL((conv_kernel<BF16, false, V, W, true>), grid, dim3(NT), 0, stream, p, nchb, ntc);
  } else {
    if (yf) hipLaunchKernelGGL((conv_kernel<BF16, true, V, W, false>), grid, dim3(NT), 0, stream, p, nchb, ntc);
    else hipLaunchKernelGGL((conv_kernel<BF16, false, V, W, false>), grid, dim3(NT), 0, stream, p, nchb, ntc);
  }
}

template <bool BF16, int V>
void launch_v(const ConvParams& p, hipStream_t stream) {
  switch (p.W) {
    case 1: launch_w<BF16, V, 1>(p, stream); break;
    case 2: launch_w<BF16, V, 2>(p, stream); break;
    case 3: launch_w<BF16, V, 3>(p, stream); break;
    case 4: launch_w<BF16, V, 4>(p, stream); break;
    case 5: launch_w<BF16, V, 5>(p, stream); break;
    case 6: launch_w<BF16, V, 6>(p, stream); break;
    case 7: launch_w<BF16, V, 7>(p, stream); break;
    default: launch_w<BF16, V, 8>(p, stream); break;
  }
}

template <bool BF16>
void launch_io(const ConvParams& p, hipStream_t stream) {
  const int64_t e = BF16 ? 2 : 4, ye = (p.y_f32 || !BF16) ? 4 : 2;
  auto al = [](const void* ptr, int64_t bytes) { return ((uintptr_t)ptr % (uintptr_t)bytes) == 0; };
  const bool vec = p.D % 4 == 0 && al(p.x, 4 * e) && al(p.y, 4 * ye) && p.xs_b % 4 == 0 && p.xs_t % 4 == 0 &&
                   p.ys_b % 4 == 0 && p.ys_t % 4 == 0;
  if (vec) launch_v<BF16, 4>(p, stream);
  else launch_v<BF16, 1>(p, stream);
}

}  // namespace

hipError_t launch_causal_conv1d(const ConvParams& p, hipStream_t stream) {
  if (p.io_bf16) launch_io<true>(p, stream);
  else launch_io<false>(p, stream);
  return hipGetLastError();
}

}  // namespace ssm
