// Gather of raster-ordered video tokens into the padded 3-D tile order the
// forward consumes, and the scatter back ("[kernel] Extract VSA utility
// functions into fastvideo_kernel", Summary: tile partition and its inverse,
// variable block sizes, non-pad index).
//
// HBM-bound copies.  One workgroup per (tile, video, head); one thread per
// 16-byte chunk of a token row (rows whose length is a multiple of 8 bf16
// values) or per element (e.g. a per-token gate); the tile-order side is
// written (gather) or read (scatter) contiguously, the raster side in runs of
// the tile's w extent.  Padding slots of a tile are written with zeros by the
// gather and ignored by the scatter.
#include "vsa_internal.hpp"

namespace vsa {
namespace {

constexpr int kCopyThreads = 256;

// One workgroup per (tile, video, head): the tile's geometry is worked out
// once, then the blk slots x copy units of the tile are spread over the
// threads (32-bit index arithmetic only).
template <bool VEC>
__global__ __launch_bounds__(kCopyThreads) void tile_copy_kernel(TileGrid G, const uint16_t* __restrict__ src,
                                                                 uint16_t* __restrict__ dst, int B, int Hh,
                                                                 int elems, int scatter) {
    const int cpr = VEC ? elems / 8 : elems;  // copy units per row
    const int tile = blockIdx.x % G.ntiles;
    const int bh = blockIdx.x / G.ntiles;     // video b, head h
    const int b = bh % B, h = bh / B;
    int et, eh, ew;
    const int size = tile_extents(G, tile, et, eh, ew);
    const int64_t P = (int64_t)G.blk * G.ntiles;
    const int64_t S = (int64_t)G.T * G.H * G.W;
    const int64_t tiled0 = ((int64_t)h * B + b) * P + (int64_t)G.blk * tile;  // row of slot 0
    const int64_t raster0 = ((int64_t)b * Hh + h) * S;
    for (int i = threadIdx.x; i < G.blk * cpr; i += kCopyThreads) {
        const int u = i / cpr, c = i - u * cpr;
        const int64_t tiled = tiled0 + u;
        if (u >= size) {
            if (!scatter) {
                if (VEC)
                    *reinterpret_cast<uint4*>(dst + tiled * elems + 8 * c) = make_uint4(0, 0, 0, 0);
                else
                    dst[tiled * elems + c] = 0;
            }
            continue;
        }
        const int64_t raster = raster0 + tile_token_raster(G, tile, u, eh, ew);
        const int64_t from = (scatter ? tiled : raster) * elems, to = (scatter ? raster : tiled) * elems;
        if (VEC)
            *reinterpret_cast<uint4*>(dst + to + 8 * c) = *reinterpret_cast<const uint4*>(src + from + 8 * c);
        else
            dst[to + c] = src[from + c];
    }
}

}  // namespace

hipError_t launch_tile_copy(const TileGrid& g, const uint16_t* src, uint16_t* dst, int B, int Hh, int elems,
                            bool scatter, hipStream_t st) {
    const int64_t wgs = (int64_t)g.ntiles * B * Hh;
    if (wgs <= 0 || wgs > 0x7fffffff) return hipErrorInvalidValue;
    if (elems % 8 == 0)
        hipLaunchKernelGGL(tile_copy_kernel<true>, dim3((unsigned)wgs), dim3(kCopyThreads), 0, st, g, src, dst, B,
                           Hh, elems, (int)scatter);
    else
        hipLaunchKernelGGL(tile_copy_kernel<false>, dim3((unsigned)wgs), dim3(kCopyThreads), 0, st, g, src, dst, B,
                           Hh, elems, (int)scatter);
    return hipGetLastError();
}

}  // namespace vsa
