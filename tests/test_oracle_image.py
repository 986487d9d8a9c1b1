"""The oracle's saved session image against its pins."""
import oracle
import pins
from oracle import kvq8_oracle as o


def test_image_pins():
    pins.pin_image(o.save_image, o.load_image, oracle.Cache, o.cache_bytes,
                   o.FMT_F16, o.FMT_Q8, o.FMT_K8V4)
