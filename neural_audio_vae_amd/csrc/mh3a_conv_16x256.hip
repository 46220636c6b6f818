// Conv kernel instances of the 16 x 256 tile shape (see mh3a_conv.h).
#include "mh3a_conv.h"

namespace mh3a {

template <>
hipError_t launch_tile_of<TILE_16x256>(const ConvArgs& a, hipStream_t stream) {
    return launch_tile16(a, stream);
}

}  // namespace mh3a
