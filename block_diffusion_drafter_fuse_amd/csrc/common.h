// Shared device helpers for the gfx950 kernels: storage types, MFMA steps,
// 16-byte loads, per-call request metadata passed by value.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dfl {

typedef uint16_t bf16_t;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMaxReq = 64;     // requests per call
constexpr int kMaxLayers = 16;  // drafter layers
constexpr int kMaxSeg = 40;     // weight segments of one virtual GEMM operand
constexpr int kMaxKSeg = 16;    // activation segments along K (tapped layers)
constexpr int kVTile = 32;      // keys per V^T tile of the context cache ([hd][kVTile] per tile)

__device__ __forceinline__ float bf2f(bf16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ __forceinline__ bf16_t f2bf(float f) {
  __bf16 b = (__bf16)f;  // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(bf16_t, b);
}

template <typename T> __device__ __forceinline__ float to_f(T v);
template <> __device__ __forceinline__ float to_f<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f<bf16_t>(bf16_t v) { return bf2f(v); }

template <typename T> __device__ __forceinline__ T from_f(float v);
template <> __device__ __forceinline__ float from_f<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f<bf16_t>(float v) { return f2bf(v); }

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// Streaming (read-once) 16-byte load: weights are used once per launch.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_stream(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// One MFMA "k-step": each lane supplies 16 bytes of a 16-row A fragment and
// 16 bytes of a 16-column B fragment; lane l covers row/column (l & 15) and
// k-group (l >> 4).  Both operands use the same k placement, so the pairing of
// k indices across lanes is consistent whatever order the hardware reduces in.
// C layout (16x16 fp32): lane l holds C[4*(l>>4) + i][l & 15], i = 0..3.
template <typename T> struct Mma;

template <> struct Mma<bf16_t> {
  static constexpr int KSTEP = 32;  // bf16 elements per k-step (8 per lane)
  static constexpr int EPL = 8;     // elements per lane per k-step
  __device__ __forceinline__ static f32x4_t step(uint4 a, uint4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
};

template <> struct Mma<float> {
  static constexpr int KSTEP = 16;  // fp32 elements per k-step (4 per lane, 4 MFMAs)
  static constexpr int EPL = 4;
  __device__ __forceinline__ static f32x4_t step(uint4 a, uint4 b, f32x4_t c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
    return c;
  }
};

// Request metadata of one draft call (block rows m = r*B + j).
struct DraftMeta {
  int n_req;
  int B;
  int ctx[kMaxReq];   // fused context length of request r (block starts there)
};

// Request metadata of one fuse call (rows grouped by request).
struct FuseMeta {
  int n_req;
  int row0[kMaxReq + 1];  // first row of request r in the call
  int pos0[kMaxReq];      // absolute position of that row
  int slot[kMaxReq];
};

__device__ __forceinline__ int fuse_req_of_row(const FuseMeta& fm, int m) {
  int r = 0;
  while (r + 1 < fm.n_req && m >= fm.row0[r + 1]) ++r;
  return r;
}

// Request metadata of one relay call (relay rows grouped by request).
struct RelayMeta {
  int n_req;
  int row0[kMaxReq + 1];  // first relay row of request r
  int slot[kMaxReq];
  int nacc[kMaxReq];      // accepted candidates of request r's round
};

__device__ __forceinline__ int relay_req_of_row(const RelayMeta& rm, int m) {
  int r = 0;
  while (r + 1 < rm.n_req && m >= rm.row0[r + 1]) ++r;
  return r;
}

// Relay rows a draft call reads: for request r, rows[(slot[r]*B + j)*D] hold
// the inputs of block offsets j = 2 .. 1 + n[r] (n[r] = 0: none).
struct DraftRelay {
  const float* rows;
  int slot[kMaxReq];
  int n[kMaxReq];
};

__device__ __forceinline__ float silu(float x) { return x / (1.0f + __expf(-x)); }

// Combine a value with the one in lane l ^ 16 (l ^ 32) with the gfx950 lane
// swaps (VALU, no LDS round trip): each returns both halves of the lane pair,
// and max / + of the two is the same in both lanes (commutative).
__device__ __forceinline__ float xor16_max(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float xor32_max(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float xor16_sum(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

}  // namespace dfl
