// Conv kernel instances of the 128x160 (row-block waves) tile shape (see mh3a_conv.h).
#include "mh3a_conv.h"

namespace mh3a {

MH3A_DEFINE_TILE_LAUNCHER(TILE_128x160R, 1, 5, 4, 1)

}  // namespace mh3a
