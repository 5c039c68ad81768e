// Gather of raster-ordered video tokens into the padded 3-D tile order the
// forward consumes, and the scatter back ("[kernel] Extract VSA utility
// functions into fastvideo_kernel", Summary: tile partition and its inverse,
// variable block sizes, non-pad index).
//
// HBM-bound copies.  One thread per 16-byte chunk of a token row (rows whose
// length is a multiple of 8 bf16 values) or per element (e.g. a per-token
// gate); the tile-order side is written (gather) or read (scatter)
// contiguously, the raster side in runs of the tile's w extent.  Padding
// slots of a tile are written with zeros by the gather and ignored by the
// scatter.
#include "vsa_internal.hpp"

namespace vsa {
namespace {

constexpr int kCopyThreads = 256;

template <bool VEC>
__global__ __launch_bounds__(kCopyThreads) void tile_copy_kernel(TileGrid G, const uint16_t* __restrict__ src,
                                                                 uint16_t* __restrict__ dst, int B, int Hh,
                                                                 int elems, int scatter, int64_t items) {
    const int cpr = VEC ? elems / 8 : elems;  // copy units per row
    const int64_t P = (int64_t)kBlock * G.ntiles;
    const int64_t S = (int64_t)G.T * G.H * G.W;
    for (int64_t it = (int64_t)blockIdx.x * kCopyThreads + threadIdx.x; it < items;
         it += (int64_t)gridDim.x * kCopyThreads) {
        const int c = (int)(it % cpr);
        int64_t rest = it / cpr;
        const int64_t slot = rest % P;
        rest /= P;
        const int b = (int)(rest % B);
        const int h = (int)(rest / B);
        const int tile = (int)(slot / kBlock), u = (int)(slot % kBlock);
        int et, eh, ew;
        const int size = tile_extents(G, tile, et, eh, ew);
        const int64_t tiled = ((int64_t)h * B + b) * P + slot;  // row in the tile-order tensor
        if (u >= size) {
            if (!scatter) {
                if (VEC)
                    *reinterpret_cast<uint4*>(dst + tiled * elems + 8 * c) = make_uint4(0, 0, 0, 0);
                else
                    dst[tiled * elems + c] = 0;
            }
            continue;
        }
        const int64_t raster = ((int64_t)b * Hh + h) * S + tile_token_raster(G, tile, u, eh, ew);
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
    const bool vec = elems % 8 == 0;
    const int64_t items = (int64_t)Hh * B * kBlock * g.ntiles * (vec ? elems / 8 : elems);
    if (items <= 0) return hipErrorInvalidValue;
    const int64_t want = (items + kCopyThreads - 1) / kCopyThreads;
    const unsigned blocks = (unsigned)(want < 65536 ? want : 65536);
    if (vec)
        hipLaunchKernelGGL(tile_copy_kernel<true>, dim3(blocks), dim3(kCopyThreads), 0, st, g, src, dst, B, Hh,
                           elems, (int)scatter, items);
    else
        hipLaunchKernelGGL(tile_copy_kernel<false>, dim3(blocks), dim3(kCopyThreads), 0, st, g, src, dst, B, Hh,
                           elems, (int)scatter, items);
    return hipGetLastError();
}

}  // namespace vsa
