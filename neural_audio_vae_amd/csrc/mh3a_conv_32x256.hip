// Conv kernel instances of the 32x256 tile shape (see mh3a_conv.h).
#include "mh3a_conv.h"

namespace mh3a {

MH3A_DEFINE_TILE_LAUNCHER(TILE_32x256, 1, 2, 1, 4)

}  // namespace mh3a
