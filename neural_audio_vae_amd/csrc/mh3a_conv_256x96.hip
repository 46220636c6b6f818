// Conv kernel instances of the 256x96 tile shape (see mh3a_conv.h).
#include "mh3a_conv.h"

namespace mh3a {

MH3A_DEFINE_TILE_LAUNCHER(TILE_256x96, 2, 3, 4, 1)

}  // namespace mh3a
