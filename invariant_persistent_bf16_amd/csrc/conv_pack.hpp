// Lowering of a 2-D convolution to the batched GEMM: the per-sample unfold of
// "Batch-Invariant VLAs" (section "Replacing nn.Conv2d") and "Batch-Invariant
// Kernel Design ..." (section "Kernel 1: Conv2d"), written out explicitly.
//
//   weight pack: Wp[co][k] = w[co][ci][kh][kw] with k = ci*Kh*Kw + kh*Kw + kw,
//                zero for Kg <= k < Kp (Kg = Cin/G*Kh*Kw, Kp = Kg rounded up to 8)
//   unfold:      U[n][g][l][k] = x[n][g*Cin/G + ci][oh*sh + kh*dh - ph][ow*sw + kw*dw - pw]
//                (zero outside the image and for k >= Kg), l = oh*OW + ow
//
// U is stored K-contiguous per location, which is the layout the GEMM's B
// operand reads directly; the product per (sample, group) is then
// y[n, g*Cout/G : (g+1)*Cout/G, :] = Wp_g @ U[n][g]^T-view, written in NCHW.
// Both kernels only move data; every arithmetic step stays in the GEMM.
#pragma once

#include "common.hpp"

namespace bi {

struct ConvGeom {
    int64_t N, Cin, H, W, Cout, Kh, Kw, sh, sw, ph, pw, dh, dw, groups;
    int64_t OH, OW, L, cig, cog, Kg, Kp;
};

// The same geometry in 32-bit fields, for shapes whose every index (input,
// unfold and packed-weight elements) is below 2^31.
struct ConvGeom32 {
    int N, Cin, H, W, Cout, Kh, Kw, sh, sw, ph, pw, dh, dw, groups;
    int OW, L, cig, Kg, Kp;
};

template <typename T>
__device__ __forceinline__ void store8(T* dst, const T (&v)[8]) {
    if constexpr (sizeof(T) == 2) {
        u32x4_t w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (uint32_t)v[2 * e] | ((uint32_t)v[2 * e + 1] << 16);
        *(u32x4_t*)dst = w;
    } else {
        *(f32x4_t*)dst = f32x4_t{v[0], v[1], v[2], v[3]};
        *(f32x4_t*)(dst + 4) = f32x4_t{v[4], v[5], v[6], v[7]};
    }
}

// Weight pack and unfold with 32-bit indices, in one launch (at one image
// each is only a few microseconds of work, less than a launch's fixed cost):
// work item i < Cout * Kp/8 packs 8 consecutive k of one co row; the others
// unfold 8 consecutive k of one (n, g, l) row of U.  For the unfold, k0 is
// split into (ci, kh, kw) once; the 8 elements then advance kw, kh, ci by
// carries, with no division per element.  One 16-byte (or two) store per item.
template <typename T>
__global__ void __launch_bounds__(256) conv_prepare32(const T* __restrict__ w, T* __restrict__ wp,
                                                     const T* __restrict__ x, T* __restrict__ u, ConvGeom32 g) {
    const int nchunk = g.Kp / 8;
    const int wtotal = g.Cout * nchunk;
    const int total = wtotal + g.N * g.groups * g.L * nchunk;
    const int khw = g.Kh * g.Kw;
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < total; i += gridDim.x * blockDim.x) {
        T v[8];
        if (i < wtotal) {
            const int co = i / nchunk, k0 = (i - co * nchunk) * 8;
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = k0 + e < g.Kg ? w[co * g.Kg + k0 + e] : (T)0;
            store8(wp + co * g.Kp + k0, v);
            continue;
        }
        int r = (i - wtotal) / nchunk;
        const int k0 = (i - wtotal - r * nchunk) * 8;
        const int l = r % g.L;
        r /= g.L;
        const int grp = r % g.groups;
        const int n = r / g.groups;
        const int oh = l / g.OW, ow = l - oh * g.OW;
        int ci = k0 / khw;
        const int rem = k0 - ci * khw;
        int kh = rem / g.Kw, kw = rem - kh * g.Kw;
        const int cbase = n * g.Cin + grp * g.cig;
        const int ih0 = oh * g.sh - g.ph, iw0 = ow * g.sw - g.pw;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            T val = (T)0;
            if (k0 + e < g.Kg) {
                const int ih = ih0 + kh * g.dh, iw = iw0 + kw * g.dw;
                if (ih >= 0 && ih < g.H && iw >= 0 && iw < g.W) val = x[((cbase + ci) * g.H + ih) * g.W + iw];
            }
            v[e] = val;
            if (++kw == g.Kw) {
                kw = 0;
                if (++kh == g.Kh) { kh = 0; ++ci; }
            }
        }
        store8(u + ((n * g.groups + grp) * g.L + l) * g.Kp + k0, v);
    }
}

// The same weight pack and unfold for the common patch geometry (16-bit
// data, no padding, no dilation, one group, Kw, the column stride and W
// even): every pair of consecutive k lies in one kernel row and starts at an
// even input column, so a 16-byte piece of U (8 consecutive k) is four
// aligned 32-bit loads.  Where each k of a piece lies relative to the
// location's first input element is a function of the piece index alone: the
// workgroup tabulates it in LDS once (koff, -1 for k >= Kg), so a piece costs
// three divisions by constants (as multiply-high by host-computed magic
// numbers, exact for the numerators the host admits), four loads and one
// 16-byte store.  Same values as conv_prepare32.
struct ConvPatch16 {
    int Cin, H, W, L, OW, sh, sw, Kh, Kw, Kg, Kp;
    int nchunk;           // Kp / 8 pieces per row
    int wchunks, total;   // weight pieces (first), all pieces
    uint64_t m_nchunk, m_L, m_OW;   // ceil(2^32 / d): floor(x / d) = (x * m) >> 32
};

__device__ __forceinline__ uint32_t conv_mdiv(uint32_t x, uint64_t m) {
    return (uint32_t)(((uint64_t)x * m) >> 32);
}

__global__ void __launch_bounds__(256) conv_prepare_patch16(const uint16_t* __restrict__ w, uint16_t* __restrict__ wp,
                                                            const uint16_t* __restrict__ x, uint16_t* __restrict__ u,
                                                            ConvPatch16 g) {
    extern __shared__ __attribute__((aligned(16))) int koff[];   // [nchunk * 4]
    const int khw = g.Kh * g.Kw;
    for (int j = threadIdx.x; j < g.nchunk * 4; j += blockDim.x) {
        const int k = 2 * j;                 // piece j / 4, 32-bit word j % 4
        const int ci = k / khw, rem = k - ci * khw, kh = rem / g.Kw, kw = rem - kh * g.Kw;
        koff[j] = k < g.Kg ? (ci * g.H + kh) * g.W + kw : -1;
    }
    __syncthreads();
    const uint32_t* x32 = (const uint32_t*)x;
    const uint32_t* w32 = (const uint32_t*)w;
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < g.total; i += gridDim.x * blockDim.x) {
        u32x4_t v;
        if (i < g.wchunks) {
            const int co = (int)conv_mdiv((uint32_t)i, g.m_nchunk), c = i - co * g.nchunk;
            const int k0 = 8 * c;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = k0 + 2 * e < g.Kg ? w32[(co * g.Kg + k0) / 2 + e] : 0u;
            *(u32x4_t*)(wp + co * g.Kp + k0) = v;
            continue;
        }
        const int r = i - g.wchunks;
        const int row = (int)conv_mdiv((uint32_t)r, g.m_nchunk), c = r - row * g.nchunk;
        const int n = (int)conv_mdiv((uint32_t)row, g.m_L), l = row - n * g.L;
        const int oh = (int)conv_mdiv((uint32_t)l, g.m_OW), ow = l - oh * g.OW;
        const int base = (n * g.Cin * g.H + oh * g.sh) * g.W + ow * g.sw;   // even
        const int4 ko = *(const int4*)&koff[4 * c];
        v[0] = ko.x >= 0 ? x32[(base + ko.x) / 2] : 0u;
        v[1] = ko.y >= 0 ? x32[(base + ko.y) / 2] : 0u;
        v[2] = ko.z >= 0 ? x32[(base + ko.z) / 2] : 0u;
        v[3] = ko.w >= 0 ? x32[(base + ko.w) / 2] : 0u;
        *(u32x4_t*)(u + row * g.Kp + 8 * c) = v;
    }
}

// The patch geometry again, one workgroup per output row (n, oh): the input
// rows oh*sh .. oh*sh + Kh - 1 of every channel are Kh*W consecutive elements
// of x, and U's rows (n, oh*OW .. oh*OW + OW - 1) are OW*Kp consecutive
// elements, so the workgroup reads Cin such blocks with 16-byte loads into
// LDS and writes its OW rows of U with 16-byte stores, each piece gathered
// from LDS as four aligned 32-bit words (offsets tabulated per piece as in
// conv_prepare_patch16).  Each thread of the grid also packs one piece of the
// weight (the grid holds at least as many threads as pieces).  Needs, besides the patch
// geometry, 16-byte aligned x and channel / row-block / row-stride sizes in
// whole 16-byte pieces (checked on the host).  Same values as conv_prepare32.
struct ConvPatchRows {
    int Cin, H, W, OH, OW, sh, sw, Kh, Kw, Kg, Kp;
    int nchunk;           // Kp / 8 pieces per row of U
    int blk;              // Kh * W: elements of one channel's input rows
    int pieces;           // blk / 8
    int wchunks;          // Cout * nchunk weight pieces
    int rowblocks;        // N * OH workgroups unfold; the grid may hold more, which only pack weight
    uint64_t m_nchunk, m_pieces;   // ceil(2^32 / d): floor(x / d) = (x * m) >> 32
};

__global__ void __launch_bounds__(256) conv_prepare_patch_rows(const uint16_t* __restrict__ w, uint16_t* __restrict__ wp,
                                                               const uint16_t* __restrict__ x, uint16_t* __restrict__ u,
                                                               ConvPatchRows g) {
    extern __shared__ __attribute__((aligned(16))) int smem[];
    int* koff = smem;                                    // [nchunk * 4]: word offset of k pair inside the blocks, -1 past Kg
    uint32_t* xs = (uint32_t*)(smem + g.nchunk * 4);     // [Cin][Kh][W] bf16 as words
    const int tid = threadIdx.x;

    // this thread's weight piece (one per thread of the grid): loads issued with the input's
    const uint32_t* w32 = (const uint32_t*)w;
    const int wi = blockIdx.x * 256 + tid;
    u32x4_t wv = {0u, 0u, 0u, 0u};
    int wco = 0, wk0 = 0;
    if (wi < g.wchunks) {
        wco = (int)conv_mdiv((uint32_t)wi, g.m_nchunk);
        wk0 = 8 * (wi - wco * g.nchunk);
#pragma unroll
        for (int e = 0; e < 4; ++e) wv[e] = wk0 + 2 * e < g.Kg ? w32[(wco * g.Kg + wk0) / 2 + e] : 0u;
    }
    if ((int)blockIdx.x >= g.rowblocks) {   // uniform over the workgroup
        if (wi < g.wchunks) *(u32x4_t*)(wp + wco * g.Kp + wk0) = wv;
        return;
    }
    const int n = blockIdx.x / g.OH, oh = blockIdx.x - n * g.OH;

    // the Cin row blocks, 16-byte pieces, up to 6 per thread in flight
    const int nl = g.Cin * g.pieces;
    const uint16_t* xb = x + ((int64_t)n * g.Cin * g.H + (int64_t)oh * g.sh) * g.W;
    for (int j0 = tid; j0 < nl; j0 += 6 * 256) {
        u32x4_t v[6];
#pragma unroll
        for (int r = 0; r < 6; ++r) {
            const int j = j0 + 256 * r;
            if (j < nl) {
                const int ci = (int)conv_mdiv((uint32_t)j, g.m_pieces), q = j - ci * g.pieces;
                v[r] = *(const u32x4_t*)(xb + (int64_t)ci * g.H * g.W + 8 * q);
            }
        }
#pragma unroll
        for (int r = 0; r < 6; ++r) {
            const int j = j0 + 256 * r;
            if (j < nl) *(u32x4_t*)(xs + 4 * j) = v[r];   // channel blocks back to back: ci * blk + 8 q
        }
    }
    const int khw = g.Kh * g.Kw;
    for (int j = tid; j < g.nchunk * 4; j += 256) {
        const int k = 2 * j;
        const int ci = k / khw, rem = k - ci * khw, kh = rem / g.Kw, kw = rem - kh * g.Kw;
        koff[j] = k < g.Kg ? (ci * g.blk + kh * g.W + kw) / 2 : -1;
    }
    if (wi < g.wchunks) *(u32x4_t*)(wp + wco * g.Kp + wk0) = wv;
    __syncthreads();

    // OW rows of U, consecutive: piece j is row ow = j / nchunk, k = 8 (j mod nchunk)
    uint16_t* dst = u + ((int64_t)n * g.OH + oh) * g.OW * g.Kp;
    for (int j = tid; j < g.OW * g.nchunk; j += 256) {
        const int ow = (int)conv_mdiv((uint32_t)j, g.m_nchunk), c = j - ow * g.nchunk;
        const int col = ow * g.sw / 2;
        const int4 ko = *(const int4*)&koff[4 * c];
        u32x4_t v;
        v[0] = ko.x >= 0 ? xs[ko.x + col] : 0u;
        v[1] = ko.y >= 0 ? xs[ko.y + col] : 0u;
        v[2] = ko.z >= 0 ? xs[ko.z + col] : 0u;
        v[3] = ko.w >= 0 ? xs[ko.w + col] : 0u;
        *(u32x4_t*)(dst + 8 * j) = v;
    }
}

// One thread per 8 consecutive k of one (co) row.
template <typename T>
__global__ void conv_pack_weight(const T* __restrict__ w, T* __restrict__ wp, ConvGeom g) {
    const int64_t nchunk = g.Kp / 8;
    const int64_t total = g.Cout * nchunk;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t co = i / nchunk, k0 = (i - co * nchunk) * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int64_t k = k0 + e;
            wp[co * g.Kp + k] = k < g.Kg ? w[co * g.Kg + k] : (T)0;
        }
    }
}

// One thread per 8 consecutive k of one (n, g, l) row of U.
template <typename T>
__global__ void conv_unfold(const T* __restrict__ x, T* __restrict__ u, ConvGeom g) {
    const int64_t nchunk = g.Kp / 8;
    const int64_t total = g.N * g.groups * g.L * nchunk;
    const int64_t khw = g.Kh * g.Kw;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        int64_t r = i / nchunk;
        const int64_t k0 = (i - r * nchunk) * 8;
        const int64_t l = r % g.L;
        r /= g.L;
        const int64_t grp = r % g.groups;
        const int64_t n = r / g.groups;
        const int64_t oh = l / g.OW, ow = l - (l / g.OW) * g.OW;
        T* dst = u + ((n * g.groups + grp) * g.L + l) * g.Kp + k0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int64_t k = k0 + e;
            T v = (T)0;
            if (k < g.Kg) {
                const int64_t ci = k / khw, rem = k - (k / khw) * khw;
                const int64_t kh = rem / g.Kw, kw = rem - (rem / g.Kw) * g.Kw;
                const int64_t ih = oh * g.sh + kh * g.dh - g.ph;
                const int64_t iw = ow * g.sw + kw * g.dw - g.pw;
                if (ih >= 0 && ih < g.H && iw >= 0 && iw < g.W)
                    v = x[((n * g.Cin + grp * g.cig + ci) * g.H + ih) * g.W + iw];
            }
            dst[e] = v;
        }
    }
}

}  // namespace bi
