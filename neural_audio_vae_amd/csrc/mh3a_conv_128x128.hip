// Conv kernel instances of the 128x128 tile shape (see mh3a_conv.h).
#include "mh3a_conv.h"

namespace mh3a {

MH3A_DEFINE_TILE_LAUNCHER(TILE_128x128, 2, 2, 2, 2)

}  // namespace mh3a
