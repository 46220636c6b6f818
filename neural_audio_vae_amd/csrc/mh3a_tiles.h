// Per-tile-shape launchers of the conv kernel. Each is defined in a
// translation unit of its own (mh3a_conv_<tile>.hip) so that the many
// instances of the kernel compile in parallel.
#pragma once

#include "mh3a_internal.h"

namespace mh3a {

template <TileId T>
hipError_t launch_tile_of(const ConvArgs& a, hipStream_t stream);
#define MH3A_TILE(id, mbw, nbw, wm, wn) template <> hipError_t launch_tile_of<id>(const ConvArgs&, hipStream_t);
MH3A_TILE_LIST
#undef MH3A_TILE
template <> hipError_t launch_tile_of<TILE_16x256>(const ConvArgs&, hipStream_t);

}  // namespace mh3a
