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
// step is one contiguous row segment.
#include <hip/hip_runtime.h>

#include "ssm_internal.h"

namespace ssm {
namespace {

constexpr int NT = 256;
constexpr int TS = 32;  // time steps per thread
constexpr float kLog2e = 1.4426950408889634f;

template <bool BF16, int V>
struct Row {
  uint32_t w[BF16 ? (V + 1) / 2 : V];
};

template <bool BF16, int V>
__device__ __forceinline__ Row<BF16, V> load_row(const void* x, int64_t off) {
  Row<BF16, V> r;
  if constexpr (BF16 && V == 4) {
    const uint2 v = *(const uint2*)((const uint16_t*)x + off);
    r.w[0] = v.x; r.w[1] = v.y;
  } else if constexpr (!BF16 && V == 4) {
    const uint4 v = *(const uint4*)((const float*)x + off);
    r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
  } else if constexpr (BF16) {
    r.w[0] = ((const uint16_t*)x)[off];
  } else {
    r.w[0] = ((const uint32_t*)x)[off];
  }
  return r;
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

template <bool BF16, int V>
__device__ __forceinline__ void store_row(const ConvParams& p, int64_t off, const float (&o)[V]) {
  if (p.y_f32 || !BF16) {
    if constexpr (V == 4) *(float4*)((float*)p.y + off) = make_float4(o[0], o[1], o[2], o[3]);
    else ((float*)p.y)[off] = o[0];
  } else {
    if constexpr (V == 4) {
      uint2 w;
      w.x = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o[0]) |
            ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o[1]) << 16);
      w.y = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o[2]) |
            ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o[3]) << 16);
      *(uint2*)((uint16_t*)p.y + off) = w;
    } else {
      ((__bf16*)p.y)[off] = (__bf16)o[0];
    }
  }
}

template <bool BF16, int V, int W>
__global__ __launch_bounds__(NT) void conv_kernel(ConvParams p, unsigned nchb, unsigned ntc) {
  const unsigned blk = blockIdx.x;
  const unsigned cg = blk % nchb;
  const unsigned tc = (blk / nchb) % ntc;
  const int64_t b = blk / (nchb * ntc);
  const int64_t d0 = ((int64_t)cg * NT + threadIdx.x) * V;
  if (d0 >= p.D) return;  // V divides D on the vector path, so a thread is all in or all out
  const int64_t t0 = (int64_t)tc * TS;

  float wv[V][W], bv[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
#pragma unroll
    for (int k = 0; k < W; ++k) wv[v][k] = p.w[(d0 + v) * p.ws_d + k * p.ws_k];
    bv[v] = p.bias ? p.bias[(d0 + v) * p.bs_d] : 0.f;
  }
  // the run and its W - 1 predecessors; steps outside [0, L) read a valid row
  // (clamped) and are zeroed after the load, so no load sits behind a branch
  constexpr int R = TS + W - 1;
  Row<BF16, V> rows[R];
  const int64_t xb = b * p.xs_b + d0;
#pragma unroll
  for (int j = 0; j < R; ++j) {
    int64_t t = t0 - (W - 1) + j;
    t = t < 0 ? 0 : (t >= p.L ? p.L - 1 : t);
    rows[j] = load_row<BF16, V>(p.x, xb + t * p.xs_t);
  }
  const int64_t yb = b * p.ys_b + d0;
#pragma unroll
  for (int j = 0; j < TS; ++j) {
    const int64_t t = t0 + j;
    float o[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      float acc = bv[v];
#pragma unroll
      for (int k = 0; k < W; ++k) {
        const int64_t ts = t - (W - 1) + k;
        const float xv = ts >= 0 ? elem<BF16, V>(rows[j + k], v) : 0.f;
        acc = __builtin_fmaf(wv[v][k], xv, acc);
      }
      if (p.silu) acc *= __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-acc * kLog2e));
      o[v] = acc;
    }
    if (t < p.L) store_row<BF16, V>(p, yb + t * p.ys_t, o);
  }
}

template <bool BF16, int V, int W>
void launch_w(const ConvParams& p, hipStream_t stream) {
  const unsigned nchb = (unsigned)((p.D + (int64_t)NT * V - 1) / ((int64_t)NT * V));
  const unsigned ntc = (unsigned)((p.L + TS - 1) / TS);
  const dim3 grid(nchb * ntc * (unsigned)p.batch);
  hipLaunchKernelGGL((conv_kernel<BF16, V, W>), grid, dim3(NT), 0, stream, p, nchb, ntc);
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
