// Conv kernel instances of the tile shapes without compile-time tap counts (see mh3a_conv.h).
#include "mh3a_conv.h"

namespace mh3a {

MH3A_DEFINE_TILE_LAUNCHER(TILE_512x64, 4, 2, 4, 1)
MH3A_DEFINE_TILE_LAUNCHER(TILE_256x128, 2, 4, 4, 1)
MH3A_DEFINE_TILE_LAUNCHER(TILE_128x256, 2, 4, 2, 2)
MH3A_DEFINE_TILE_LAUNCHER(TILE_64x512, 2, 4, 1, 4)
MH3A_DEFINE_TILE_LAUNCHER(TILE_32x512, 1, 4, 1, 4)

}  // namespace mh3a
