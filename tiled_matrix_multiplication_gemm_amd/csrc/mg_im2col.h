// im2col for gfx950: the data movement that turns a 2-D convolution into the
// GEMM of this library (FlagOS cross-chip page, section 5.3: convolution is
// lowered to a GEMM through im2col and reuses the GEMM's optimisations).
//
// Input x is NHWC [Nb,H,W,C]; the result `cols` is [M = Nb*OH*OW, ld] with
// row m = (n*OH + oh)*OW + ow holding, at column k = (kh*KW + kw)*C + c, the
// input value x[n, oh*sh - ph + kh*dh, ow*sw - pw + kw*dw, c], or zero where
// that position lies outside the image; columns K = KH*KW*C .. ld-1 are zero.
//
// The work is bound by HBM (it reads x up to KH*KW times and writes cols
// once), so both kernels move whole 16-byte chunks, coalesced along C:
//  * im2col_tap_kernel (C a multiple of the 16-byte vector, ld == K): one
//    kernel tap (kh, kw) per blockIdx.y and a run of output rows per
//    blockIdx.x.  Each row's (n, oh*sh - ph, ow*sw - pw) is decoded once into
//    LDS; each chunk then costs one 32-bit division (row within the run) and
//    one 16-byte load (or a zero) and store.  Consecutive lanes walk the C
//    run of one input pixel, so loads and stores are contiguous.
//  * im2col_elem_kernel (any C): the same row runs over whole chunks of the
//    ld-wide row, each of the chunk's elements decoded on its own.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace mg {

struct Im2colArgs {
    const char* x;
    char* cols;
    int64_t H, W, C;   // input height, width, channels
    int64_t M, K, ld;  // output rows, used columns, row stride (elements)
    int32_t KH, KW, sh, sw, ph, pw, dh, dw, OH, OW;
    int32_t rows_per_block;
};

inline constexpr int kIm2colThreads = 256;
inline constexpr int kIm2colMaxRows = 256;

struct Im2colRow {
    int64_t base;  // element offset of image n
    int32_t ih0, iw0;
};

// Decode rows m0 .. m0+rows-1 into LDS (one row per thread).
__device__ __forceinline__ void im2col_rows(const Im2colArgs& a, int64_t m0, int rows, Im2colRow* sr) {
    for (int r = threadIdx.x; r < rows; r += kIm2colThreads) {
        const uint32_t m = (uint32_t)(m0 + r);  // the host keeps M below 2^31
        const uint32_t ohw = (uint32_t)a.OH * (uint32_t)a.OW;
        const uint32_t n = m / ohw, rem = m - n * ohw;
        const uint32_t oh = rem / (uint32_t)a.OW, ow = rem - oh * (uint32_t)a.OW;
        sr[r].base = (int64_t)n * a.H * a.W * a.C;
        sr[r].ih0 = (int32_t)oh * a.sh - a.ph;
        sr[r].iw0 = (int32_t)ow * a.sw - a.pw;
    }
    __syncthreads();
}

template <int ES>
__global__ __launch_bounds__(kIm2colThreads) void im2col_tap_kernel(const Im2colArgs a) {
    constexpr int V = 16 / ES;
    __shared__ Im2colRow sr[kIm2colMaxRows];
    const int64_t m0 = (int64_t)blockIdx.x * a.rows_per_block;
    const int rows = (int)((a.M - m0) < a.rows_per_block ? (a.M - m0) : a.rows_per_block);
    im2col_rows(a, m0, rows, sr);
    const int tap = blockIdx.y;
    const int kh = tap / a.KW, kw = tap - kh * a.KW;
    const int dh = kh * a.dh, dw = kw * a.dw;
    const uint32_t cv = (uint32_t)(a.C / V);  // chunks per input pixel
    const uint32_t total = (uint32_t)rows * cv;
    for (uint32_t idx = threadIdx.x; idx < total; idx += kIm2colThreads) {
        const uint32_t r = idx / cv, cc = idx - r * cv;
        const int ih = sr[r].ih0 + dh, iw = sr[r].iw0 + dw;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (ih >= 0 && ih < a.H && iw >= 0 && iw < a.W)
            v = *(const uint4*)(a.x + (sr[r].base + ((int64_t)ih * a.W + iw) * a.C + (int64_t)cc * V) * ES);
        *(uint4*)(a.cols + ((m0 + r) * a.ld + (int64_t)tap * a.C + (int64_t)cc * V) * ES) = v;
    }
}

template <int ES>
__global__ __launch_bounds__(kIm2colThreads) void im2col_elem_kernel(const Im2colArgs a) {
    constexpr int V = 16 / ES;
    using Elem = typename std::conditional<ES == 2, uint16_t, uint32_t>::type;
    __shared__ Im2colRow sr[kIm2colMaxRows];
    const int64_t m0 = (int64_t)blockIdx.x * a.rows_per_block;
    const int rows = (int)((a.M - m0) < a.rows_per_block ? (a.M - m0) : a.rows_per_block);
    im2col_rows(a, m0, rows, sr);
    const uint32_t lc = (uint32_t)(a.ld / V);  // chunks per output row
    const uint32_t total = (uint32_t)rows * lc;
    const Elem* x = (const Elem*)a.x;
    for (uint32_t idx = threadIdx.x; idx < total; idx += kIm2colThreads) {
        const uint32_t r = idx / lc, kc = idx - r * lc;
        union {
            uint4 v;
            Elem e[V];
        } u;
#pragma unroll
        for (int j = 0; j < V; ++j) {
            const uint32_t k = kc * V + j;  // the host keeps ld below 2^27
            Elem e = 0;
            if (k < (uint32_t)a.K) {
                const uint32_t tap = k / (uint32_t)a.C, c = k - tap * (uint32_t)a.C;
                const int kh = (int)(tap / (uint32_t)a.KW), kw = (int)(tap - (uint32_t)kh * (uint32_t)a.KW);
                const int ih = sr[r].ih0 + kh * a.dh, iw = sr[r].iw0 + kw * a.dw;
                if (ih >= 0 && ih < a.H && iw >= 0 && iw < a.W) e = x[sr[r].base + ((int64_t)ih * a.W + iw) * a.C + c];
            }
            u.e[j] = e;
        }
        *(uint4*)(a.cols + ((m0 + r) * a.ld + (int64_t)kc * V) * ES) = u.v;
    }
}

}  // namespace mg
