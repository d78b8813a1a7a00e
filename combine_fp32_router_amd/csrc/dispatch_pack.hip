// Dispatch pack: stable scatter of hidden rows into the send buffer, plain
// bf16 or per-token dynamic int8 / int4.
//
// What it computes (aggregation by destination into one contiguous buffer,
// ThunderEP write-up s2.1; per-token dynamic int8 with one run-time scale per
// token, s2.3): for each slot s with pos[s] >= 0, record pos[s] = token
// s/k's row, copied bit for bit (bf16) or as H codes + fp32 scale + 12 zero
// bytes (int8; scale = max|x|/127, code = rne(x/scale) clamped to +-127; fp8
// the same with scale = max|x|/448 and an OCP E4M3 code, the NCCL EP
// article's FP8 communication, s6.3), or
// as H/2 bytes of 4-bit codes + fp32 scale + 12 zero bytes (int4, the
// write-up's 4-bit follow-up, s5.2; scale = max|x|/7, codes clamped to +-7,
// element 2i in the low nibble of byte i).
//
// gfx950 design.  One block per token; the row is read from HBM once, kept in
// VGPRs (each thread owns `VPT` 16-byte vectors, strided by the block size so
// every wave instruction moves 1 KiB of contiguous memory) and written to
// the token's k rows.  The k row numbers arrive with one vector load (lane j
// holds slot j's row) issued beside the row load and are read back with
// v_readlane, instead of k dependent scalar loads in the store loop (which
// the resident waves already hid: the two forms measured the same).
// Stores go through the cache hierarchy (not nontemporal): when one chunk's
// send buffer fits the 256 MB Infinity Cache, its consumer (the exchange, or
// combine on one device) reads it from there; measured neutral when it does
// not fit, and 11% faster for pack + combine at 8 chunks of the
// T=16384, H=7168, k=8 batch.
// The int8 variant gives each thread 16 elements, reduces max|x| over the
// block (wave shuffles + LDS), quantises in registers and stores 16 codes
// per lane (one 16-byte store per row); thread 0 writes the 16-byte scale
// slot.  Nothing here is a contraction: the kernel
// is bound by HBM write bandwidth (k row writes per row read).
#include "common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

template <int VPT>
__global__ __launch_bounds__(1024) void pack_bf16_kernel(const u32x4 *__restrict__ x, int HV,
                                                         int k, const int32_t *__restrict__ pos,
                                                         u32x4 *__restrict__ send)
{
    const int64_t t = blockIdx.x;
    const int nthr = blockDim.x;
    const u32x4 *xr = x + t * HV;
    const int32_t rows = load_per_lane(pos + t * k, k);  // lane j: row of slot j
    u32x4 v[VPT];
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        const int c = threadIdx.x + i * nthr;
        if (c < HV)
            v[i] = xr[c];  // cached load: measured faster than a streaming load here
    }
    for (int j = 0; j < k; ++j) {
        const int32_t p = lane_value(rows, j);
        if (p < 0)
            continue;
        u32x4 *dst = send + static_cast<int64_t>(p) * HV;
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int c = threadIdx.x + i * nthr;
            if (c < HV)
                dst[c] = v[i];
        }
    }
}

// int8 / fp8 (FP8 = true): each thread owns VPT groups of 16 elements (two
// 16-byte bf16 loads, one 16-byte store of 16 one-byte codes per row),
// strided by the block size.
template <int VPT, bool FP8>
__global__ __launch_bounds__(1024) void pack_byte_kernel(const u32x4 *__restrict__ x, int G,
                                                         int k, const int32_t *__restrict__ pos,
                                                         uint8_t *__restrict__ send,
                                                         int64_t stride)
{
    __shared__ float red[16];
    const int64_t t = blockIdx.x;
    const int nthr = blockDim.x;
    const u32x4 *xr = x + t * 2 * G;
    const int32_t rows = load_per_lane(pos + t * k, k);  // lane j: row of slot j
    float f[VPT][16];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        const int g = threadIdx.x + i * nthr;
        u32x4 a = u32x4{0, 0, 0, 0}, b = u32x4{0, 0, 0, 0};
        if (g < G) {
            a = xr[2 * g];
            b = xr[2 * g + 1];
        }
        unpack8(a, f[i]);
        unpack8(b, f[i] + 8);
#pragma unroll
        for (int q = 0; q < 16; ++q)
            amax = fmaxf(amax, fabsf(f[i][q]));
    }
    amax = block_max_nonneg(amax, red);
    const bool zero = (amax == 0.0f);
    const float scale = zero ? 0.0f : amax / (FP8 ? 448.0f : 127.0f);
    u32x4 codes[VPT];
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        if (FP8) {
            codes[i] = u32x4{fp8x4(f[i], scale, zero), fp8x4(f[i] + 4, scale, zero),
                             fp8x4(f[i] + 8, scale, zero), fp8x4(f[i] + 12, scale, zero)};
        } else {
            const u32x2 lo = quant8(f[i], scale, zero);
            const u32x2 hi = quant8(f[i] + 8, scale, zero);
            codes[i] = u32x4{lo.x, lo.y, hi.x, hi.y};
        }
    }

    const int H = G * 16;
    for (int j = 0; j < k; ++j) {
        const int32_t p = lane_value(rows, j);
        if (p < 0)
            continue;
        uint8_t *rec = send + static_cast<int64_t>(p) * stride;
        u32x4 *dst = reinterpret_cast<u32x4 *>(rec);
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int g = threadIdx.x + i * nthr;
            if (g < G)
                dst[g] = codes[i];
        }
        if (threadIdx.x == 0)
            *reinterpret_cast<u32x4 *>(rec + H) = u32x4{__float_as_uint(scale), 0u, 0u, 0u};
    }
}

// int4: each thread owns VPT groups of 32 elements (four 16-byte bf16 loads,
// one 16-byte store of 32 codes per row), strided by the block size.  The
// record's scale slot follows its H/2 code bytes.
template <int VPT>
__global__ __launch_bounds__(1024) void pack_int4_kernel(const u32x4 *__restrict__ x, int G,
                                                         int k, const int32_t *__restrict__ pos,
                                                         uint8_t *__restrict__ send,
                                                         int64_t stride)
{
    __shared__ float red[16];
    const int64_t t = blockIdx.x;
    const int nthr = blockDim.x;
    const u32x4 *xr = x + t * 4 * G;
    const int32_t rows = load_per_lane(pos + t * k, k);  // lane j: row of slot j
    float f[VPT][32];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        const int g = threadIdx.x + i * nthr;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const u32x4 a = (g < G) ? xr[4 * g + q] : u32x4{0, 0, 0, 0};
            unpack8(a, f[i] + 8 * q);
        }
#pragma unroll
        for (int q = 0; q < 32; ++q)
            amax = fmaxf(amax, fabsf(f[i][q]));
    }
    amax = block_max_nonneg(amax, red);
    const bool zero = (amax == 0.0f);
    const float scale = zero ? 0.0f : amax / 7.0f;
    u32x4 codes[VPT];
#pragma unroll
    for (int i = 0; i < VPT; ++i)
        codes[i] = u32x4{quant4x8(f[i], scale, zero), quant4x8(f[i] + 8, scale, zero),
                         quant4x8(f[i] + 16, scale, zero), quant4x8(f[i] + 24, scale, zero)};

    for (int j = 0; j < k; ++j) {
        const int32_t p = lane_value(rows, j);
        if (p < 0)
            continue;
        u32x4 *dst = reinterpret_cast<u32x4 *>(send + static_cast<int64_t>(p) * stride);
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int g = threadIdx.x + i * nthr;
            if (g < G)
                dst[g] = codes[i];
        }
        if (threadIdx.x == 0)
            dst[G] = u32x4{__float_as_uint(scale), 0u, 0u, 0u};
    }
}

}  // namespace

RowTiling row_tiling(int vecs)
{
    RowTiling r;
    r.vpt = 1;
    while (r.vpt < 8 && (vecs + r.vpt - 1) / r.vpt > 1024)
        r.vpt *= 2;
    int thr = (vecs + r.vpt - 1) / r.vpt;
    thr = ((thr + kWave - 1) / kWave) * kWave;
    r.threads = thr < kWave ? kWave : thr;
    return r;
}

hipError_t launch_dispatch_pack(const void *x, int64_t T, int H, int k, const int32_t *pos,
                                int quant, void *send, hipStream_t stream)
{
    const int HV = H / 8;
    const RowTiling rt = row_tiling(HV);
    const dim3 grid(static_cast<unsigned>(T));
    const dim3 block(rt.threads);
    const u32x4 *xv = static_cast<const u32x4 *>(x);
    if (quant == 0) {
        u32x4 *sv = static_cast<u32x4 *>(send);
        switch (rt.vpt) {
        case 1: pack_bf16_kernel<1><<<grid, block, 0, stream>>>(xv, HV, k, pos, sv); break;
        case 2: pack_bf16_kernel<2><<<grid, block, 0, stream>>>(xv, HV, k, pos, sv); break;
        case 4: pack_bf16_kernel<4><<<grid, block, 0, stream>>>(xv, HV, k, pos, sv); break;
        default: pack_bf16_kernel<8><<<grid, block, 0, stream>>>(xv, HV, k, pos, sv); break;
        }
    } else if (quant == 1 || quant == 3) {
        uint8_t *sb = static_cast<uint8_t *>(send);
        const int64_t stride = record_bytes(H, quant);
        const int G = H / 16;
        const RowTiling gt = row_tiling(G);
        const dim3 gblock(gt.threads);
        if (quant == 1) {
            switch (gt.vpt) {
            case 1: pack_byte_kernel<1, false><<<grid, gblock, 0, stream>>>(xv, G, k, pos, sb, stride); break;
            case 2: pack_byte_kernel<2, false><<<grid, gblock, 0, stream>>>(xv, G, k, pos, sb, stride); break;
            case 4: pack_byte_kernel<4, false><<<grid, gblock, 0, stream>>>(xv, G, k, pos, sb, stride); break;
            default: pack_byte_kernel<8, false><<<grid, gblock, 0, stream>>>(xv, G, k, pos, sb, stride); break;
            }
        } else {
            switch (gt.vpt) {
            case 1: pack_byte_kernel<1, true><<<grid, gblock, 0, stream>>>(xv, G, k, pos, sb, stride); break;
            case 2: pack_byte_kernel<2, true><<<grid, gblock, 0, stream>>>(xv, G, k, pos, sb, stride); break;
            case 4: pack_byte_kernel<4, true><<<grid, gblock, 0, stream>>>(xv, G, k, pos, sb, stride); break;
            default: pack_byte_kernel<8, true><<<grid, gblock, 0, stream>>>(xv, G, k, pos, sb, stride); break;
            }
        }
    } else {
        uint8_t *sb = static_cast<uint8_t *>(send);
        const int64_t stride = record_bytes(H, 2);
        const int G = H / 32;
        const RowTiling gt = row_tiling(G);
        const dim3 gblock(gt.threads);
        switch (gt.vpt) {
        case 1: pack_int4_kernel<1><<<grid, gblock, 0, stream>>>(xv, G, k, pos, sb, stride); break;
        case 2: pack_int4_kernel<2><<<grid, gblock, 0, stream>>>(xv, G, k, pos, sb, stride); break;
        case 4: pack_int4_kernel<4><<<grid, gblock, 0, stream>>>(xv, G, k, pos, sb, stride); break;
        default: pack_int4_kernel<8><<<grid, gblock, 0, stream>>>(xv, G, k, pos, sb, stride); break;
        }
    }
    return hipGetLastError();
}

}  // namespace moe
