// Device helpers shared by the gfx950 kernels of the dispatch/combine path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;  // CDNA wavefront width

// Payload formats of a row: 0 bf16 (2H bytes), 1 int8 (H codes), 2 int4
// (H/2 bytes, two codes per byte), 3 fp8 (H OCP E4M3 codes).  A quantised
// row's fp32 scale is not stored in the row but at the same index of a
// separate scale array, so rows stay whole 128-byte lines when H is a
// multiple of 128 (bf16: 64; int4: 256).
__host__ __device__ inline int64_t row_bytes(int H, int quant)
{
    return quant == 0 ? 2 * static_cast<int64_t>(H)
                      : (quant == 2 ? static_cast<int64_t>(H) / 2 : static_cast<int64_t>(H));
}

// Native clang vectors: 16-byte and 8-byte global accesses
// (global_load/store_dwordx4 / dwordx2), usable with the nontemporal builtins.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Device-scope stores (cache policy sc1) through a raw buffer descriptor
// over one row: the row's bytes are written through the XCD's L2 to the
// memory side, where the last-level cache keeps them for their consumer,
// instead of leaving dirty lines in L2 until eviction.  The descriptor is
// built from a wave-uniform row address (scalar registers); `bytes` bounds
// the row, and a lane's offset is in bytes from the row start.
constexpr int kRawBufferWord3 = 0x00020000;  // raw (untyped) 32-bit elements
constexpr int kCpolDevice = 16;               // sc1: device scope
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(void *row, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(row, 0, bytes, kRawBufferWord3);
}
__device__ __forceinline__ void store_device(__amdgpu_buffer_rsrc_t r, int off, u32x4 v)
{
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kCpolDevice);
}
__device__ __forceinline__ void store_device(__amdgpu_buffer_rsrc_t r, int off, u32x2 v)
{
    __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, kCpolDevice);
}

// Streaming device-scope stores (nt + sc1): written through to memory
// without being kept in the last-level cache.  The pack uses them when its
// output is not read back soon from this GPU (MOE_PACK_STREAM): the cache
// then holds no dirty send rows that other traffic must evict and write back.
constexpr int kCpolStreamDevice = 2 | kCpolDevice;
template <bool STREAM>
__device__ __forceinline__ void store_row(__amdgpu_buffer_rsrc_t r, int off, u32x4 v)
{
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, STREAM ? kCpolStreamDevice : kCpolDevice);
}
template <bool STREAM>
__device__ __forceinline__ void store_row(__amdgpu_buffer_rsrc_t r, int off, u32x2 v)
{
    __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, STREAM ? kCpolStreamDevice : kCpolDevice);
}

// Row loads through a raw buffer descriptor (see row_rsrc).  An offset at
// or past the descriptor's size reads zeros, so lanes past the row's end and
// rows described with size 0 (a dropped slot) need no predicate.
constexpr int kCpolDefault = 0;
constexpr int kCpolStream = 2;  // nontemporal (slc)
__device__ __forceinline__ u32x4 load_cached(__amdgpu_buffer_rsrc_t r, int off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCpolDefault);
}
__device__ __forceinline__ u32x2 load_stream8(__amdgpu_buffer_rsrc_t r, int off)
{
    return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kCpolStream);
}
__device__ __forceinline__ u32x4 load_stream16(__amdgpu_buffer_rsrc_t r, int off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCpolStream);
}


// A value every lane of the wave holds identically, made visibly uniform so
// the compiler keeps it in SGPRs and uses scalar loads for what it indexes.
__device__ __forceinline__ uint32_t uniform(uint32_t v)
{
    return __builtin_amdgcn_readfirstlane(v);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// The n (<= 64) int32 values v[0..n-1], one per lane (lane j holds v[j],
// -1 past n): one vector load per wave instead of n dependent scalar loads.
// Read element j back with lane_value(x, j).
__device__ __forceinline__ int32_t load_per_lane(const int32_t *__restrict__ v, int n)
{
    const int lane = lane_id();
    return lane < n ? v[lane] : -1;
}

__device__ __forceinline__ float load_per_lane(const float *__restrict__ v, int n)
{
    const int lane = lane_id();
    return lane < n ? v[lane] : 0.0f;
}

// Value of lane j (wave-uniform j) as a wave-uniform scalar.
__device__ __forceinline__ int32_t lane_value(int32_t x, int j)
{
    return __builtin_amdgcn_readlane(x, j);
}

__device__ __forceinline__ float lane_value(float x, int j)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), j));
}

// bf16 halves of a 32-bit word -> fp32 (exact widening).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    const __bf16 a = static_cast<__bf16>(lo);
    const __bf16 b = static_cast<__bf16>(hi);
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, a)) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b)) << 16);
}

// 8 bf16 (one 16-byte vector) -> 8 fp32
__device__ __forceinline__ void unpack8(const u32x4 v, float f[8])
{
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
    f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
    f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

__device__ __forceinline__ u32x4 pack8(const float f[8])
{
    u32x4 v;
    v.x = pack_bf16x2(f[0], f[1]);
    v.y = pack_bf16x2(f[2], f[3]);
    v.z = pack_bf16x2(f[4], f[5]);
    v.w = pack_bf16x2(f[6], f[7]);
    return v;
}

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1)
        v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

// --- DPP (data-parallel primitives): cross-lane moves inside the VALU, no
// LDS traffic.  Controls used (GFX9 encoding): quad_perm [1,0,3,2] = 0xB1,
// quad_perm [2,3,0,1] = 0x4E, row_half_mirror = 0x141, row_mirror = 0x140.
// Applied in that order with a commutative operator they leave every lane of
// a 16-lane row holding the row's reduction.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp32(uint32_t v)
{
    return static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, false));
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp64(uint64_t v)
{
    const uint32_t lo = dpp32<CTRL>(static_cast<uint32_t>(v));
    const uint32_t hi = dpp32<CTRL>(static_cast<uint32_t>(v >> 32));
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint64_t row_max_u64(uint64_t v)
{
    v = umax64(v, dpp64<0xB1>(v));
    v = umax64(v, dpp64<0x4E>(v));
    v = umax64(v, dpp64<0x141>(v));
    v = umax64(v, dpp64<0x140>(v));
    return v;
}

__device__ __forceinline__ uint64_t readlane64(uint64_t v, int lane)
{
    const uint32_t lo = static_cast<uint32_t>(
        __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v)), lane));
    const uint32_t hi = static_cast<uint32_t>(
        __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v >> 32)), lane));
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Max of a 64-bit key over the wave, returned wave-uniform (scalar): DPP row
// reductions, then the four row results read into SGPRs.
__device__ __forceinline__ uint64_t wave_max_u64_dpp(uint64_t v)
{
    v = row_max_u64(v);
    return umax64(umax64(readlane64(v, 0), readlane64(v, 16)),
                  umax64(readlane64(v, 32), readlane64(v, 48)));
}

// Sum of a double over one 16-lane row; every lane of the row gets it.
__device__ __forceinline__ double row_sum_f64(double v)
{
    auto step = [](double x, uint64_t y) { return x + __longlong_as_double(static_cast<long long>(y)); };
    v = step(v, dpp64<0xB1>(static_cast<uint64_t>(__double_as_longlong(v))));
    v = step(v, dpp64<0x4E>(static_cast<uint64_t>(__double_as_longlong(v))));
    v = step(v, dpp64<0x141>(static_cast<uint64_t>(__double_as_longlong(v))));
    v = step(v, dpp64<0x140>(static_cast<uint64_t>(__double_as_longlong(v))));
    return v;
}

// Inclusive prefix sum across the wave (Hillis-Steele on shuffles).
__device__ __forceinline__ int wave_inclusive_scan(int v)
{
    const int lane = lane_id();
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int u = __shfl_up(v, o);
        if (lane >= o)
            v += u;
    }
    return v;
}

// Max over the block of per-thread values >= 0; `red` holds >= 16 floats
// of LDS.  Every thread gets the result.  Contains two block barriers.
__device__ __forceinline__ float block_max_nonneg(float v, float *red)
{
    const int w = threadIdx.x / kWave;
    const int nw = (blockDim.x + kWave - 1) / kWave;
    v = wave_max(v);
    if (lane_id() == 0)
        red[w] = v;
    __syncthreads();
    float m = 0.0f;
    for (int i = 0; i < nw; ++i)
        m = fmaxf(m, red[i]);
    __syncthreads();
    return m;
}

// Per-token dynamic int8 code of one element: x / scale (IEEE fp32
// division), round half to even, clamp to [-127, 127].
__device__ __forceinline__ int quant_code(float x, float scale)
{
    float r = rintf(x / scale);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return static_cast<int>(r);
}

// 8 fp32 -> 8 int8 codes packed little-endian in a u32x2; scale == 0 -> 0.
__device__ __forceinline__ u32x2 quant8(const float f[8], float scale, bool zero)
{
    uint32_t b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        b[i] = zero ? 0u : (static_cast<uint32_t>(quant_code(f[i], scale)) & 0xffu);
    u32x2 q;
    q.x = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
    q.y = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
    return q;
}

// Per-token dynamic int4 code: x / scale (IEEE fp32 division), round half to
// even, clamp to [-7, 7].
__device__ __forceinline__ int quant_code4(float x, float scale)
{
    float r = rintf(x / scale);
    r = fminf(fmaxf(r, -7.0f), 7.0f);
    return static_cast<int>(r);
}

// 8 fp32 -> 8 int4 codes in one 32-bit word, element i in bits 4i..4i+3
// (so in memory element 2j is the low nibble of byte j); scale == 0 -> 0.
__device__ __forceinline__ uint32_t quant4x8(const float f[8], float scale, bool zero)
{
    uint32_t q = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        q |= zero ? 0u : ((static_cast<uint32_t>(quant_code4(f[i], scale)) & 0xfu) << (4 * i));
    return q;
}

// 8 int4 codes -> 8 fp32 values code * scale (fp32 multiply); each nibble is
// sign-extended by an arithmetic shift.
__device__ __forceinline__ void dequant4x8(uint32_t q, float scale, float f[8])
{
#pragma unroll
    for (int i = 0; i < 8; ++i)
        f[i] = static_cast<float>(static_cast<int32_t>(q << (28 - 4 * i)) >> 28) * scale;
}

// 8 int4 codes -> 16 * code as fp32 (exact).  Each code is masked into the
// high nibble of its own byte -- even elements from (q << 4), odd ones from
// q itself -- where the byte read as a signed integer is 16 * code, so each
// element costs one sign-extending byte convert (an SDWA operand select)
// plus a share of three mask operations per 8 codes; the caller folds the
// exact factor 1/16 into its multiplier.
__device__ __forceinline__ void codes4x8_x16(uint32_t q, float f[8])
{
    const uint32_t even = (q << 4) & 0xF0F0F0F0u;
    const uint32_t odd = q & 0xF0F0F0F0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = static_cast<float>(static_cast<int8_t>((even >> (8 * i)) & 0xffu));
        f[2 * i + 1] = static_cast<float>(static_cast<int8_t>((odd >> (8 * i)) & 0xffu));
    }
}

// fp8 (OCP E4M3): the gfx950 conversion instructions round to nearest even
// and match the format's definition on every code (checked exhaustively
// against an independent encoder).  4 fp32 -> 4 codes in a 32-bit word,
// element i in byte i; scale == 0 -> 0.
__device__ __forceinline__ uint32_t fp8x4(const float f[4], float scale, bool zero)
{
    if (zero)
        return 0u;
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(f[0] / scale, f[1] / scale, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(f[2] / scale, f[3] / scale, w, true);
    return static_cast<uint32_t>(w);
}

// 8 fp8 codes -> 8 fp32 values decode(code) * scale (fp32 multiply).
__device__ __forceinline__ void dequant_fp8x8(const u32x2 q, float scale, float f[8])
{
    const int a = static_cast<int>(q.x), b = static_cast<int>(q.y);
    f[0] = __builtin_amdgcn_cvt_f32_fp8(a, 0) * scale;
    f[1] = __builtin_amdgcn_cvt_f32_fp8(a, 1) * scale;
    f[2] = __builtin_amdgcn_cvt_f32_fp8(a, 2) * scale;
    f[3] = __builtin_amdgcn_cvt_f32_fp8(a, 3) * scale;
    f[4] = __builtin_amdgcn_cvt_f32_fp8(b, 0) * scale;
    f[5] = __builtin_amdgcn_cvt_f32_fp8(b, 1) * scale;
    f[6] = __builtin_amdgcn_cvt_f32_fp8(b, 2) * scale;
    f[7] = __builtin_amdgcn_cvt_f32_fp8(b, 3) * scale;
}

// 8 int8 codes -> 8 fp32 values code * scale (fp32 multiply).
__device__ __forceinline__ void dequant8(const u32x2 q, float scale, float f[8])
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[i] = static_cast<float>(static_cast<int8_t>((q.x >> (8 * i)) & 0xffu)) * scale;
        f[4 + i] = static_cast<float>(static_cast<int8_t>((q.y >> (8 * i)) & 0xffu)) * scale;
    }
}

}  // namespace moe
