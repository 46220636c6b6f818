// Conv kernel instances of the 64x256 tile shape (see mh3a_conv.h).
#include "mh3a_conv.h"

namespace mh3a {

MH3A_DEFINE_TILE_LAUNCHER(TILE_64x256, 2, 2, 1, 4)

}  // namespace mh3a
